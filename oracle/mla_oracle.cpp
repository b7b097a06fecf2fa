// CPU oracle for MLA decode over a paged latent cache, in C++ (test
// infrastructure: only the tests, the smoke check and the benchmark's CPU
// baseline load it; it shares no source with the GPU library).
//
// It computes the plain, unabsorbed definition in double precision.  MLA in
// the DeepSeek-V2 form that GLM-4.7-Flash uses (model record "GLM-4.7-Flash",
// config facts: MLA with kv_a_proj_with_mqa and kv_b_proj; SERVICEABILITY
// JOIN: the cache holds one shared low-rank latent c_t plus a decoupled RoPE
// key k^R_t per token).  For head h, with kv_b_proj stored per head as
// [W_UK^h (d_nope rows) ; W_UV^h (d_v rows)] over the latent width d_c:
//
//   K^h_t = [ W_UK^h c_t , k^R_t ]       (query head d_nope + d_rope wide)
//   V^h_t =   W_UV^h c_t                 (value head d_v wide)
//   s_t   = scale * < q^h , K^h_t >
//   out^h = sum_t softmax(s)_t V^h_t ,   lse^h = log sum_t exp(s_t)
//
// Query j of the Sq new tokens of a sequence of length L sees tokens
// 0 .. L - Sq + j; a query that sees none gets out = 0, lse = -inf.  Token t
// is read from page block_table[b][t / P], slot t % P.  Every K and V is
// rebuilt from the stored row for every head, and the softmax is the
// textbook two-pass one (maximum, then the sum of exponentials): pass 1
// rebuilds each key and stores its score, pass 2 rebuilds each value and
// accumulates it with its weight, so memory is O(L) per (sequence, head).
//
// Stored formats, each decoded exactly to double from its definition:
//   f32                IEEE binary32
//   bf16               the upper 16 bits of a binary32
//   fp8 e4m3 + e8m0    (model record, ENGINE KERNEL CONSTRAINTS (2), 528 B per
//                      token) n e4m3fn codes, then one e8m0 scale per 32
//                      values: value = e4m3fn * 2^(E - 127)
//   fp4 e2m1 + e4m3    (model record, SERVICEABILITY JOIN, 288 B per token;
//                      the block size and scale format are this build's
//                      reading) n/2 bytes of e2m1 codes, value 2i in the low
//                      nibble of byte i, then one e4m3fn scale per 16 values
//
// Built with g++ -O3 -fopenmp as oracle/libmla_oracle.so; parallel over
// (sequence, head) pairs.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

namespace {

enum { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP4 = 3 };

double f32_value(const uint8_t* p) {
  float f;
  std::memcpy(&f, p, 4);
  return (double)f;
}

double bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// is subnormal (m / 8 * 2^-6); S.1111.111 is NaN; no infinities.
double e4m3fn_value(uint8_t c) {
  const double s = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 0xF, m = c & 0x7;
  if (e == 0xF && m == 0x7) return std::numeric_limits<double>::quiet_NaN();
  if (e == 0) return s * (m / 8.0) * std::ldexp(1.0, -6);
  return s * (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
}

// OCP e8m0: 2^(E - 127); E = 255 is NaN.
double e8m0_value(uint8_t e) {
  if (e == 0xFF) return std::numeric_limits<double>::quiet_NaN();
  return std::ldexp(1.0, (int)e - 127);
}

// OCP e2m1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
// subnormal (m / 2).
double e2m1_value(uint8_t c) {
  const double s = (c & 0x8) ? -1.0 : 1.0;
  const int e = (c >> 1) & 0x3, m = c & 0x1;
  if (e == 0) return s * m * 0.5;
  return s * (1.0 + m / 2.0) * std::ldexp(1.0, e - 1);
}

size_t row_bytes(int fmt, int n) {
  switch (fmt) {
    case kF32: return 4 * (size_t)n;
    case kBF16: return 2 * (size_t)n;
    case kFP8: return (size_t)n + n / 32;
    case kFP4: return (size_t)n / 2 + n / 16;
  }
  return 0;
}

// One stored row of n values -> double.
void decode_row(const uint8_t* r, int fmt, int n, double* out) {
  switch (fmt) {
    case kF32:
      for (int i = 0; i < n; ++i) out[i] = f32_value(r + 4 * i);
      break;
    case kBF16:
      for (int i = 0; i < n; ++i) out[i] = bf16_value((uint16_t)(r[2 * i] | (r[2 * i + 1] << 8)));
      break;
    case kFP8:
      for (int i = 0; i < n; ++i) out[i] = e4m3fn_value(r[i]) * e8m0_value(r[n + i / 32]);
      break;
    case kFP4:
      for (int i = 0; i < n; ++i) {
        const uint8_t code = (i % 2 == 0) ? (r[i / 2] & 0xF) : (r[i / 2] >> 4);
        out[i] = e2m1_value(code) * e4m3fn_value(r[n / 2 + i / 16]);
      }
      break;
  }
}

// A q or weight tensor element stored as f32 (fmt 0) or bf16 bits (fmt 1).
double tensor_value(const void* base, int fmt, int64_t i) {
  if (fmt == 0) return (double)static_cast<const float*>(base)[i];
  return bf16_value(static_cast<const uint16_t*>(base)[i]);
}

}  // namespace

extern "C" {

// Unabsorbed MLA decode (see the top of this file).
//   q            [B*Sq][H][dn + dr], q_fmt (0 f32, 1 bf16 bits)
//   w            [H][dn + dv][dc], w_fmt
//   pool         [num_pages][P][row bytes of kv_fmt]
//   block_table  [B][max_blocks], seq_lens [B]
//   seqs         sequences to compute (n_seqs of them; NULL = all B)
//   out          [B*Sq][H][dv], lse [B*Sq][H]: written for the selected
//                sequences only
//   threads      OpenMP threads (0 = the runtime's default)
// Returns 0, or -1 if a block-table entry a sequence needs lies outside
// [0, num_pages) or a length exceeds the table (nothing is then written for
// that sequence).
int mla_oracle_decode(int B, int Sq, int H, int dn, int dr, int dv, int dc, const void* q, int q_fmt,
                      const void* w, int w_fmt, const uint8_t* pool, int kv_fmt, int64_t num_pages, int P,
                      const int32_t* block_table, int max_blocks, const int32_t* seq_lens, double scale,
                      const int32_t* seqs, int n_seqs, double* out, double* lse, int threads) {
  const int n = dc + dr;
  const size_t rb = row_bytes(kv_fmt, n);
  std::vector<int32_t> sel;
  if (seqs) sel.assign(seqs, seqs + n_seqs);
  else for (int b = 0; b < B; ++b) sel.push_back(b);

  // Per head, W_UK^h and W_UV^h transposed to [dc][dn] and [dc][dv], so that
  // W c is accumulated as a sum over c of (column c) * c_t[c]: for every
  // output element the terms are added in the order c = 0, 1, ..., dc - 1.
  std::vector<double> wuk_t((size_t)H * dc * dn), wuv_t((size_t)H * dc * dv);
  for (int h = 0; h < H; ++h)
    for (int k = 0; k < dn + dv; ++k)
      for (int c = 0; c < dc; ++c) {
        const double x = tensor_value(w, w_fmt, ((int64_t)h * (dn + dv) + k) * dc + c);
        if (k < dn) wuk_t[((size_t)h * dc + c) * dn + k] = x;
        else wuv_t[((size_t)h * dc + c) * dv + (k - dn)] = x;
      }

  // Validate the tables of the selected sequences first.
  int status = 0;
  std::vector<char> ok(sel.size(), 1);
  for (size_t i = 0; i < sel.size(); ++i) {
    const int b = sel[i];
    const int64_t L = seq_lens[b];
    if (L < 0 || L > (int64_t)max_blocks * P) { ok[i] = 0; status = -1; continue; }
    for (int64_t pg = 0; pg < (L + P - 1) / P; ++pg) {
      const int64_t phys = block_table[(int64_t)b * max_blocks + pg];
      if (phys < 0 || phys >= num_pages) { ok[i] = 0; status = -1; break; }
    }
  }

  const int64_t tasks = (int64_t)sel.size() * H;
  if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel
  {
    std::vector<double> row(n), k(dn), v(dv), o((size_t)Sq * dv), s, qd((size_t)Sq * (dn + dr));
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
      const size_t si = (size_t)(task / H);
      const int h = (int)(task % H);
      if (!ok[si]) continue;
      const int b = sel[si];
      const int64_t L = seq_lens[b];
      const double* WUK = wuk_t.data() + (size_t)h * dc * dn;
      const double* WUV = wuv_t.data() + (size_t)h * dc * dv;
      auto load_row = [&](int64_t t) {
        const int64_t phys = block_table[(int64_t)b * max_blocks + t / P];
        decode_row(pool + ((size_t)phys * P + (size_t)(t % P)) * rb, kv_fmt, n, row.data());
      };
      // Visible tokens of query j: L - Sq + 1 + j.
      auto visible = [&](int j) { return L - Sq + 1 + j; };
      s.assign((size_t)Sq * (size_t)(L > 0 ? L : 0), 0.0);
      for (int j = 0; j < Sq; ++j)
        for (int i = 0; i < dn + dr; ++i)
          qd[(size_t)j * (dn + dr) + i] = tensor_value(q, q_fmt, ((int64_t)(b * Sq + j) * H + h) * (dn + dr) + i);

      // Pass 1: K_t = [W_UK c_t, k^R_t] and the scores.
      for (int64_t t = 0; t < L; ++t) {
        load_row(t);
        for (int i = 0; i < dn; ++i) k[i] = 0.0;
        for (int c = 0; c < dc; ++c) {
          const double x = row[c];
          const double* col = WUK + (size_t)c * dn;
          for (int i = 0; i < dn; ++i) k[i] += col[i] * x;
        }
        for (int j = 0; j < Sq; ++j) {
          if (t >= visible(j)) continue;
          const double* qj = qd.data() + (size_t)j * (dn + dr);
          double dot = 0.0;
          for (int i = 0; i < dn; ++i) dot += qj[i] * k[i];
          for (int i = 0; i < dr; ++i) dot += qj[dn + i] * row[dc + i];
          s[(size_t)j * L + t] = scale * dot;
        }
      }
      // Two-pass softmax: the maximum over the visible scores ...
      std::vector<double> m(Sq, -std::numeric_limits<double>::infinity()), z(Sq, 0.0);
      for (int j = 0; j < Sq; ++j)
        for (int64_t t = 0; t < visible(j); ++t) m[j] = std::fmax(m[j], s[(size_t)j * L + t]);
      // ... then pass 2: V_t = W_UV c_t weighted by exp(s_t - m).
      for (size_t i = 0; i < o.size(); ++i) o[i] = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        if (t >= visible(Sq - 1)) break;  // no query sees token t
        load_row(t);
        for (int i = 0; i < dv; ++i) v[i] = 0.0;
        for (int c = 0; c < dc; ++c) {
          const double x = row[c];
          const double* col = WUV + (size_t)c * dv;
          for (int i = 0; i < dv; ++i) v[i] += col[i] * x;
        }
        for (int j = 0; j < Sq; ++j) {
          if (t >= visible(j)) continue;
          const double p = std::exp(s[(size_t)j * L + t] - m[j]);
          z[j] += p;
          for (int i = 0; i < dv; ++i) o[(size_t)j * dv + i] += p * v[i];
        }
      }
      for (int j = 0; j < Sq; ++j) {
        const int64_t r = (int64_t)(b * Sq + j) * H + h;
        if (visible(j) <= 0) {
          for (int i = 0; i < dv; ++i) out[r * dv + i] = 0.0;
          lse[r] = -std::numeric_limits<double>::infinity();
          continue;
        }
        for (int i = 0; i < dv; ++i) out[r * dv + i] = o[(size_t)j * dv + i] / z[j];
        lse[r] = m[j] + std::log(z[j]);
      }
    }
  }
  return status;
}

// Threads an OpenMP parallel region of this library would use.
int mla_oracle_max_threads(void) { return omp_get_max_threads(); }

}  // extern "C"
