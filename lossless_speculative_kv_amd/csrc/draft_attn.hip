// Draft decode attention over the compressed cache (VeriCache summary, "Core
// algorithm": drafting runs the target model over KV_comp; "P1": drafting is
// bound by HBM bandwidth, so the kernel streams the compressed bytes once and
// dequantises in registers).
//
// Work decomposition: one workgroup (4 waves) per (body split, KV head,
// sequence), plus one extra split per (KV head, sequence) for the
// unquantised tail. Each wave owns a contiguous run of 32-token blocks and
// keeps an online-softmax state for all g query heads of the KV head; the 4
// wave states are merged through LDS, and the per-split partials (max, sum,
// unnormalised output) are merged in split order by draft_merge_kernel.
//
// MFMA mapping (v_mfma_f32_16x16x32, fp16 for KIVI, bf16 for bf16 rows):
//   QK: S^T[token][col] = sum_k A[token][k] B[k][col] with A = key codes of
//       16 tokens and B = the scaled query. Column col = NG*hl + j packs a
//       query head (hl) with a 32-channel group j (NG = D/32 groups): in
//       K-step kk the B column is nonzero only when j == kk, so column
//       (hl, j) accumulates the partial score over channel group j and a sum
//       over the NG adjacent lanes gives the full score. This lets each lane
//       fold the key scales of one channel group only (8 channels), instead
//       of all D channels for every (padded) head.
//   PV: O^T[channel][col] = sum_t V^T[channel][t] P~[t][col] with
//       P~[t][(hl, j)] = p[t][hl] * value_scale[t][group j]; output column
//       (hl, j) is kept only for channels of group j.
//   Key scale and the 1/sqrt(D)*log2(e) factor are folded into the fp16
//   query per 32-token key group; key zero points become a per-(group, head)
//   score bias. Value zero points add sum_t p[t] * zero[t][j] per (head, j).
//
// 2/4-bit codes become fp16 MFMA operands with one AND-OR each: the code is
// masked into the mantissa of an fp16 whose exponent makes the code's least
// significant bit worth 1, so the operand equals base + code exactly (base a
// power of two). For keys the base contribution sum_k q~_k * base_k is
// subtracted through the bias; for values the base is removed with one
// packed fp16 add (exact), keeping the long fp32 accumulation small.
#include "attn_common.h"

namespace vc {

namespace {

constexpr int kWaves = 4;

struct DraftParams {
  const uint16_t* q;  // bf16 [B][Hq][D]
  float* part_o;      // [B][Hq][S][D]
  float* part_ml;     // [B][Hq][S][2]
  float* out;         // [B][Hq][D]
  int B, Hq, Hkv, g, S, bpw;
  float qscale;       // log2(e) / sqrt(D)
  int body_cap, tail_cap, src_t_cap;
  const int32_t* body_len;
  const int32_t* tail_len;
  const uint32_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint32_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  const int32_t* kept_idx;
  const uint16_t* src_k;
  const uint16_t* src_v;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
};

// ---------------------------------------------------------------- codes ----
// 2-bit word (16 codes, channel/slot f in bits 2f and 16 + 2f) -> 8 fp16x2
// registers, register f = (base_f + code_f(low half), base_f + code_f(high half)).
__device__ __forceinline__ void unpack2(uint32_t w, uint32_t (&R)[8]) {
  const uint32_t w4 = w << 4, w6 = w >> 6;
  R[0] = (w4 & 0x00300030u) | 0x54005400u;  // bits 0-1   -> mantissa 4-5, base 64
  R[1] = (w4 & 0x00C000C0u) | 0x4C004C00u;  // bits 2-3   -> mantissa 6-7, base 16
  R[2] = (w & 0x00300030u) | 0x54005400u;   // bits 4-5,  base 64
  R[3] = (w & 0x00C000C0u) | 0x4C004C00u;   // bits 6-7,  base 16
  R[4] = (w & 0x03000300u) | 0x44004400u;   // bits 8-9,  base 4
  R[5] = (w6 & 0x00300030u) | 0x54005400u;  // bits 10-11 -> 4-5, base 64
  R[6] = (w6 & 0x00C000C0u) | 0x4C004C00u;  // bits 12-13 -> 6-7, base 16
  R[7] = (w6 & 0x03000300u) | 0x44004400u;  // bits 14-15 -> 8-9, base 4
}
__device__ __forceinline__ constexpr float base2(int f) {
  return (f == 4 || f == 7) ? 4.f : ((f == 1 || f == 3 || f == 6) ? 16.f : 64.f);
}
// 4-bit word (8 codes, nibble f in bits 4f and 16 + 4f) -> 4 registers, base 64.
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t (&R)[4]) {
  R[0] = ((w << 4) & 0x00F000F0u) | 0x54005400u;
  R[1] = (w & 0x00F000F0u) | 0x54005400u;
  R[2] = ((w >> 4) & 0x00F000F0u) | 0x54005400u;
  R[3] = ((w >> 8) & 0x00F000F0u) | 0x54005400u;
}
__device__ __forceinline__ uint32_t sub_base(uint32_t r, float base) {
  const _Float16 nb = (_Float16)(-base);
  const f16x2 v = __builtin_bit_cast(f16x2, r) + f16x2{nb, nb};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T, int N>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N == 1) {
    w[0] = p[0];
  } else if constexpr (N == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0];
    w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + i);
      w[i] = v[0];
      w[i + 1] = v[1];
      w[i + 2] = v[2];
      w[i + 3] = v[3];
    }
  }
}

// Channel of slot s for the KIVI key mapping of lane group qg and K-step kk.
template <int D, int BITS>
__device__ __forceinline__ int kivi_key_channel(int qg, int kk, int s) {
  constexpr int NWL = D * BITS / 128;
  if constexpr (BITS == 2) return 16 * (qg * NWL + (kk >> 1)) + 4 * (kk & 1) + (s >> 1) + 8 * (s & 1);
  else return 8 * (qg * NWL + kk) + (s >> 1) + 4 * (s & 1);
}
// Channel of slot s for the row (unquantised) mapping.
template <int D>
__device__ __forceinline__ int row_channel(int qg, int kk, int s) {
  return qg * (D / 4) + 8 * kk + s;
}

// ------------------------------------------------------- KIVI body block ----
template <int D, int BITS, int NHS>
__device__ __forceinline__ void kivi_block(const DraftParams& P, size_t unit, int blk, int lane,
                                           const float (&qf)[NHS][8], SoftState<NHS, D / 16>& st) {
  constexpr int NG = D / 32, MT = D / 16, WPT = D * BITS / 32, NWL = D * BITS / 128, VWL = D * BITS / 64;
  const int n = lane & 15, qg = lane >> 4, j = n % NG;
  const size_t nbc = (size_t)(P.body_cap / 32);
  const size_t bidx = unit * nbc + (size_t)blk;

  // ---- loads ----
  uint32_t kw[2][NWL];
  const uint32_t* kc = P.k_codes + bidx * 32 * WPT + (size_t)qg * NWL;
  load_words<uint32_t, NWL>(kc + (size_t)n * WPT, kw[0]);
  load_words<uint32_t, NWL>(kc + (size_t)(16 + n) * WPT, kw[1]);
  uint32_t vw[VWL];
  load_words<uint32_t, VWL>(P.v_codes + (bidx * 64 + lane) * VWL, vw);

  float sk[8], zk[8];
  {
    const uint16_t* ks = P.k_scale + bidx * D;
    const uint16_t* kz = P.k_zero + bidx * D;
    if constexpr (BITS == 2) {
      const int c0 = kivi_key_channel<D, BITS>(qg, j, 0);
      const u32x2 slo = *reinterpret_cast<const u32x2*>(ks + c0), shi = *reinterpret_cast<const u32x2*>(ks + c0 + 8);
      const u32x2 zlo = *reinterpret_cast<const u32x2*>(kz + c0), zhi = *reinterpret_cast<const u32x2*>(kz + c0 + 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t wsl = slo[r >> 1], wsh = shi[r >> 1], wzl = zlo[r >> 1], wzh = zhi[r >> 1];
        sk[2 * r] = (r & 1) ? f16_hi(wsl) : f16_lo(wsl);
        sk[2 * r + 1] = (r & 1) ? f16_hi(wsh) : f16_lo(wsh);
        zk[2 * r] = (r & 1) ? f16_hi(wzl) : f16_lo(wzl);
        zk[2 * r + 1] = (r & 1) ? f16_hi(wzh) : f16_lo(wzh);
      }
    } else {
      const int c0 = kivi_key_channel<D, BITS>(qg, j, 0);
      const u32x4 sv = *reinterpret_cast<const u32x4*>(ks + c0), zv = *reinterpret_cast<const u32x4*>(kz + c0);
      // halfs 0..3 -> even slots, halfs 4..7 -> odd slots
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t a = sv[r >> 1], b = sv[2 + (r >> 1)], za = zv[r >> 1], zb = zv[2 + (r >> 1)];
        sk[2 * r] = (r & 1) ? f16_hi(a) : f16_lo(a);
        sk[2 * r + 1] = (r & 1) ? f16_hi(b) : f16_lo(b);
        zk[2 * r] = (r & 1) ? f16_hi(za) : f16_lo(za);
        zk[2 * r + 1] = (r & 1) ? f16_hi(zb) : f16_lo(zb);
      }
    }
  }
  const u32x4 vsw = *reinterpret_cast<const u32x4*>(P.v_scale + (bidx * NG + j) * 32 + qg * 8);
  const u32x4 vzw = *reinterpret_cast<const u32x4*>(P.v_zero + (bidx * NG + j) * 32 + qg * 8);

  // ---- fold key scale into the query; zero point and code base into a bias ----
  uint32_t Bq[NHS][4];
  float bias[NHS];
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    float bp = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t pr = pack_f16(qf[h][2 * r] * sk[2 * r], qf[h][2 * r + 1] * sk[2 * r + 1]);
      Bq[h][r] = pr;
      const float base = (BITS == 2) ? base2(4 * (j & 1) + r) : 64.f;
      bp += qf[h][2 * r] * zk[2 * r] + qf[h][2 * r + 1] * zk[2 * r + 1];
      bp -= (f16_lo(pr) + f16_hi(pr)) * base;
    }
    bias[h] = sum_q(sum_group<NG>(bp));
  }

  // ---- scores ----
  float s[NHS][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t A[NG][4];
    if constexpr (BITS == 2) {
#pragma unroll
      for (int wi = 0; wi < NWL; ++wi) {
        uint32_t R[8];
        unpack2(kw[i][wi], R);
#pragma unroll
        for (int f = 0; f < 8; ++f) A[2 * wi + (f >> 2)][f & 3] = R[f];
      }
    } else {
#pragma unroll
      for (int wi = 0; wi < NWL; ++wi) {
        uint32_t R[4];
        unpack4(kw[i][wi], R);
#pragma unroll
        for (int f = 0; f < 4; ++f) A[wi][f] = R[f];
      }
    }
#pragma unroll
    for (int h = 0; h < NHS; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const bool on = (j == kk);
        const u32x4 b = {on ? Bq[h][0] : 0u, on ? Bq[h][1] : 0u, on ? Bq[h][2] : 0u, on ? Bq[h][3] : 0u};
        c = mfma_f16(u32x4{A[kk][0], A[kk][1], A[kk][2], A[kk][3]}, b, c);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[h][i][r] = sum_group<NG>(c[r]) + bias[h];
    }
  }

  softmax_block<NHS, MT>(st, s);

  // ---- P~ = p * value_scale (fp16), zero-point term ----
  uint32_t Bp[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r >> 1, rr = 2 * (r & 1);
      const f16x2 ph = as_f16x2(pack_f16(s[h][i][rr], s[h][i][rr + 1]));
      const uint32_t zw = vzw[r], sw = vsw[r];
      st.zt[h] = __builtin_amdgcn_fdot2(ph, as_f16x2(zw), st.zt[h], false);
      Bp[h][r] = as_u32(ph * as_f16x2(sw));
    }

  // ---- PV ----
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
    if constexpr (BITS == 2) {
      uint32_t R[8];
      unpack2(vw[m >> 1], R);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[r] = sub_base(R[4 * (m & 1) + r], base2(4 * (m & 1) + r));
    } else {
      uint32_t R[4];
      unpack4(vw[m], R);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[r] = sub_base(R[r], 64.f);
    }
#pragma unroll
    for (int h = 0; h < NHS; ++h)
      st.acc[h][m] = mfma_f16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Bp[h][0], Bp[h][1], Bp[h][2], Bp[h][3]},
                              st.acc[h][m]);
  }
}

// ------------------------------------------------ unquantised row block ----
// A 32-token block of 16-bit rows (fp16 KIVI tail, or bf16 rows for token
// drop / dense). rows.k(t) / rows.v(t) give the row pointers of token
// t < nvalid. The query operand Bq is unscaled (exact in fp16 and bf16);
// scores are scaled by log2(e)/sqrt(D) after the MFMA.
// lds: this wave's staging area, 32 rows of D halfs with a stride of D + 4.
template <int D, int NHS, bool BF16, typename RowFn>
__device__ __forceinline__ void row_block(const RowFn& rows, int nvalid, int lane, float qscale,
                                          const uint32_t (&Bq)[NHS][4], SoftState<NHS, D / 16>& st,
                                          uint16_t* lds) {
  constexpr int NG = D / 32, MT = D / 16, LSTR = D + 4;
  const int n = lane & 15, qg = lane >> 4, j = n % NG;

  // ---- stage V rows in LDS (invalid rows as zeros) ----
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
      const int t = lane / CPR + RPI * u, c = lane % CPR;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < nvalid) v = *reinterpret_cast<const u32x4*>(rows.v(t) + 8 * c);
      uint32_t* d = reinterpret_cast<uint32_t*>(lds + t * LSTR + 8 * c);
      *reinterpret_cast<u32x2*>(d) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(d + 2) = u32x2{v[2], v[3]};
    }
  }

  // ---- scores ----
  float s[NHS][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 16 * i + n;
    uint32_t A[NG][4];
    if (t < nvalid) {
      const uint16_t* kp = rows.k(t) + qg * (D / 4);
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(kp + 8 * kk);
        A[kk][0] = v[0];
        A[kk][1] = v[1];
        A[kk][2] = v[2];
        A[kk][3] = v[3];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) A[kk][0] = A[kk][1] = A[kk][2] = A[kk][3] = 0u;
    }
#pragma unroll
    for (int h = 0; h < NHS; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const bool on = (j == kk);
        const u32x4 b = {on ? Bq[h][0] : 0u, on ? Bq[h][1] : 0u, on ? Bq[h][2] : 0u, on ? Bq[h][3] : 0u};
        c = mfma16<BF16>(u32x4{A[kk][0], A[kk][1], A[kk][2], A[kk][3]}, b, c);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum_group<NG>(c[r]) * qscale;
        s[h][i][r] = (16 * i + 4 * qg + r < nvalid) ? v : kNegInf;
      }
    }
  }

  softmax_block<NHS, MT>(st, s);

  uint32_t Bp[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r >> 1, rr = 2 * (r & 1);
      Bp[h][r] = pack16<BF16>(s[h][i][rr], s[h][i][rr + 1]);
    }

  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t lo = lds[slot_token(qg, 2 * r) * LSTR + 16 * m + n];
      const uint32_t hi = lds[slot_token(qg, 2 * r + 1) * LSTR + 16 * m + n];
      A[r] = lo | (hi << 16);
    }
#pragma unroll
    for (int h = 0; h < NHS; ++h)
      st.acc[h][m] = mfma16<BF16>(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Bp[h][0], Bp[h][1], Bp[h][2], Bp[h][3]},
                                  st.acc[h][m]);
  }
}

// The lane's 8 query values (times `scale`) for a slot -> channel mapping.
template <int D, int NHS, typename ChanFn>
__device__ __forceinline__ void load_q(const DraftParams& P, int b, int hk, int lane, float scale, ChanFn chan,
                                       float (&qf)[NHS][8]) {
  constexpr int NG = D / 32, HS = 16 / NG;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const int head = h * HS + hl;
    const bool ok = head < P.g;
    const uint16_t* qp = P.q + ((size_t)b * P.Hq + (size_t)hk * P.g + (ok ? head : 0)) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[h][s] = ok ? bf16_bits_to_f32(qp[chan(qg, j, s)]) * scale : 0.f;
  }
}

// Merge the 4 wave states of the workgroup and store the split's partial.
// lds must hold kWaves * NH * (D + 2) floats; it may alias the row staging
// area (the leading barrier orders the reuse).
template <int D, int NHS>
__device__ __forceinline__ void store_partial(const DraftParams& P, int b, int hk, int split, int lane, int wave,
                                              SoftState<NHS, D / 16>& st, bool has_zero, float* lds) {
  constexpr int NG = D / 32, HS = 16 / NG, NH = NHS * HS;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
  float* lds_o = lds;
  float* lds_ml = lds + kWaves * NH * D;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const float l = sum_q(st.l[h]);
    const float zt = has_zero ? sum_q(st.zt[h]) : 0.f;
    const int head = h * HS + hl;
    float* o = lds_o + ((size_t)wave * NH + head) * D;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * j + mm;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[16 * m + 4 * qg + r] = st.acc[h][m][r] + zt;
    }
    if (j == 0 && qg == 0) {
      lds_ml[(wave * NH + head) * 2] = st.m[h];
      lds_ml[(wave * NH + head) * 2 + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < P.g * D; idx += 64 * kWaves) {
    const int head = idx / D, c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_ml[(w * NH + head) * 2]);
    float O = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = lds_ml[(w * NH + head) * 2];
        if (mw != kNegInf) {
          const float a = fast_exp2(mw - M);
          O += lds_o[((size_t)w * NH + head) * D + c] * a;
          L += lds_ml[(w * NH + head) * 2 + 1] * a;
        }
      }
    }
    const size_t row = ((size_t)b * P.Hq + (size_t)hk * P.g + head) * P.S + split;
    P.part_o[row * D + c] = O;
    if (c == 0) {
      P.part_ml[row * 2] = M;
      P.part_ml[row * 2 + 1] = L;
    }
  }
}

template <int D>
struct PlainRows {
  const uint16_t *kb, *vb;
  __device__ __forceinline__ const uint16_t* k(int t) const { return kb + (size_t)t * D; }
  __device__ __forceinline__ const uint16_t* v(int t) const { return vb + (size_t)t * D; }
};
template <int D, bool GATHER>
struct SourceRows {
  const uint16_t *kb, *vb;
  const int32_t* idx;
  int t0, cap;
  __device__ __forceinline__ int pos(int t) const {
    if constexpr (GATHER) return min((int)((unsigned)idx[t0 + t]), cap - 1);
    else return t0 + t;
  }
  __device__ __forceinline__ const uint16_t* k(int t) const { return kb + (size_t)pos(t) * D; }
  __device__ __forceinline__ const uint16_t* v(int t) const { return vb + (size_t)pos(t) * D; }
};

template <int D, int NHS>
constexpr size_t draft_lds_bytes() {
  constexpr int HS = 16 / (D / 32), NH = NHS * HS;
  constexpr size_t part = (size_t)kWaves * NH * (D + 2) * sizeof(float);
  constexpr size_t rows = (size_t)kWaves * 32 * (D + 4) * sizeof(uint16_t);
  return part > rows ? part : rows;
}

// ---------------------------------------------------------------- kernels ----
template <int D, int BITS, int NHS>
__global__ __launch_bounds__(256) void draft_kivi_kernel(const DraftParams P) {
  constexpr int MT = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[draft_lds_bytes<D, NHS>()];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;

  SoftState<NHS, MT> st;
  st.init();
  const bool tail_split = (split == P.S - 1);
  if (!tail_split) {
    float qf[NHS][8];
    load_q<D, NHS>(P, b, hk, lane, P.qscale,
                   [](int qg_, int kk, int s) { return kivi_key_channel<D, BITS>(qg_, kk, s); }, qf);
    const int nblk = min(max(P.body_len[b], 0), P.body_cap) / 32;
    const int b0 = (split * kWaves + wave) * P.bpw;
    const int b1 = min(b0 + P.bpw, nblk);
    for (int blk = b0; blk < b1; ++blk) kivi_block<D, BITS, NHS>(P, unit, blk, lane, qf, st);
  } else {
    float qf[NHS][8];
    load_q<D, NHS>(P, b, hk, lane, 1.f, [](int qg_, int kk, int s) { return row_channel<D>(qg_, kk, s); }, qf);
    uint32_t Bq[NHS][4];
#pragma unroll
    for (int h = 0; h < NHS; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) Bq[h][r] = pack_f16(qf[h][2 * r], qf[h][2 * r + 1]);
    const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
    const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
    const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
    uint16_t* my_lds = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 4);
    for (int blk = wave; blk * 32 < nt; blk += kWaves) {
      const PlainRows<D> rows{tk + (size_t)blk * 32 * D, tv + (size_t)blk * 32 * D};
      row_block<D, NHS, false>(rows, min(32, nt - blk * 32), lane, P.qscale, Bq, st, my_lds);
    }
  }
  store_partial<D, NHS>(P, b, hk, split, lane, wave, st, !tail_split, reinterpret_cast<float*>(smem));
}

// Token-drop (GATHER) and dense draft caches: bf16 rows everywhere.
template <int D, int NHS, bool GATHER>
__global__ __launch_bounds__(256) void draft_rows_kernel(const DraftParams P) {
  constexpr int MT = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[draft_lds_bytes<D, NHS>()];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;

  SoftState<NHS, MT> st;
  st.init();
  float qf[NHS][8];
  load_q<D, NHS>(P, b, hk, lane, 1.f, [](int qg_, int kk, int s) { return row_channel<D>(qg_, kk, s); }, qf);
  uint32_t Bq[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) Bq[h][r] = pack_bf16(qf[h][2 * r], qf[h][2 * r + 1]);
  uint16_t* my_lds = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 4);
  if (split != P.S - 1) {
    const int nb = min(max(P.body_len[b], 0), P.body_cap);
    const int nblk = (nb + 31) / 32;
    const int b0 = (split * kWaves + wave) * P.bpw;
    const int b1 = min(b0 + P.bpw, nblk);
    const uint16_t* sk = P.src_k + unit * (size_t)P.src_t_cap * D;
    const uint16_t* sv = P.src_v + unit * (size_t)P.src_t_cap * D;
    const int32_t* kept = GATHER ? P.kept_idx + unit * (size_t)P.body_cap : nullptr;
    for (int blk = b0; blk < b1; ++blk) {
      const SourceRows<D, GATHER> rows{sk, sv, kept, blk * 32, P.src_t_cap};
      row_block<D, NHS, true>(rows, min(32, nb - blk * 32), lane, P.qscale, Bq, st, my_lds);
    }
  } else {
    const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
    const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
    const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
    for (int blk = wave; blk * 32 < nt; blk += kWaves) {
      const PlainRows<D> rows{tk + (size_t)blk * 32 * D, tv + (size_t)blk * 32 * D};
      row_block<D, NHS, true>(rows, min(32, nt - blk * 32), lane, P.qscale, Bq, st, my_lds);
    }
  }
  store_partial<D, NHS>(P, b, hk, split, lane, wave, st, false, reinterpret_cast<float*>(smem));
}

// Merge the splits of one (sequence, query head) in split order.
template <int D>
__global__ __launch_bounds__(D) void draft_merge_kernel(const DraftParams P) {
  const int c = threadIdx.x, hq = blockIdx.x, b = blockIdx.y;
  const size_t row0 = ((size_t)b * P.Hq + hq) * P.S;
  float M = kNegInf;
  for (int s = 0; s < P.S; ++s) M = fmaxf(M, P.part_ml[(row0 + s) * 2]);
  float O = 0.f, L = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < P.S; ++s) {
      const float ms = P.part_ml[(row0 + s) * 2];
      if (ms != kNegInf) {
        const float a = fast_exp2(ms - M);
        O += P.part_o[(row0 + s) * D + c] * a;
        L += P.part_ml[(row0 + s) * 2 + 1] * a;
      }
    }
  }
  P.out[((size_t)b * P.Hq + hq) * D + c] = (L > 0.f) ? O / L : 0.f;
}

template <int D>
int pick_nhs(int g) {
  constexpr int HS = 16 / (D / 32);
  return (g + HS - 1) / HS;
}

template <int D, int BITS>
void launch_kivi(const DraftParams& P, dim3 grid, hipStream_t s) {
  switch (pick_nhs<D>(P.g)) {
    case 1: hipLaunchKernelGGL((draft_kivi_kernel<D, BITS, 1>), grid, dim3(256), 0, s, P); break;
    case 2: hipLaunchKernelGGL((draft_kivi_kernel<D, BITS, 2>), grid, dim3(256), 0, s, P); break;
    case 3: hipLaunchKernelGGL((draft_kivi_kernel<D, BITS, 3>), grid, dim3(256), 0, s, P); break;
    default: hipLaunchKernelGGL((draft_kivi_kernel<D, BITS, 4>), grid, dim3(256), 0, s, P); break;
  }
}
template <int D, bool GATHER>
void launch_rows(const DraftParams& P, dim3 grid, hipStream_t s) {
  switch (pick_nhs<D>(P.g)) {
    case 1: hipLaunchKernelGGL((draft_rows_kernel<D, 1, GATHER>), grid, dim3(256), 0, s, P); break;
    case 2: hipLaunchKernelGGL((draft_rows_kernel<D, 2, GATHER>), grid, dim3(256), 0, s, P); break;
    case 3: hipLaunchKernelGGL((draft_rows_kernel<D, 3, GATHER>), grid, dim3(256), 0, s, P); break;
    default: hipLaunchKernelGGL((draft_rows_kernel<D, 4, GATHER>), grid, dim3(256), 0, s, P); break;
  }
}

}  // namespace

// Split plan shared by the workspace query and the launch.
struct DraftPlan {
  int bpw;     // body blocks per wave
  int splits;  // body splits + 1 tail split
};

DraftPlan draft_plan(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  const long long blocks = (kv.body_cap + 31) / 32;
  const long long units = (long long)sh.batch * sh.n_kv_heads;
  const long long target_waves = 4096;  // about 16 waves per CU on 256 CUs
  long long bpw = (blocks * units + target_waves - 1) / target_waves;
  if (bpw < 1) bpw = 1;
  if (bpw > 128) bpw = 128;
  const long long body_splits = (blocks + kWaves * bpw - 1) / (kWaves * bpw);
  return DraftPlan{(int)bpw, (int)body_splits + 1};
}

size_t draft_ws_bytes(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  const DraftPlan p = draft_plan(sh, kv);
  const size_t rows = (size_t)sh.batch * sh.n_q_heads * p.splits;
  return align_up(rows * sh.head_dim * sizeof(float), 256) + align_up(rows * 2 * sizeof(float), 256);
}

vc_status draft_launch(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out, void* ws,
                       hipStream_t stream) {
  const DraftPlan plan = draft_plan(sh, kv);
  DraftParams P{};
  P.q = static_cast<const uint16_t*>(q);
  const size_t rows = (size_t)sh.batch * sh.n_q_heads * plan.splits;
  P.part_o = static_cast<float*>(ws);
  P.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(rows * sh.head_dim * sizeof(float), 256));
  P.out = out;
  P.B = sh.batch;
  P.Hq = sh.n_q_heads;
  P.Hkv = sh.n_kv_heads;
  P.g = sh.n_q_heads / sh.n_kv_heads;
  P.S = plan.splits;
  P.bpw = plan.bpw;
  P.qscale = kLog2e / sqrtf((float)sh.head_dim);
  P.body_cap = kv.body_cap;
  P.tail_cap = kv.tail_cap;
  P.src_t_cap = kv.src_t_cap;
  P.body_len = kv.body_len;
  P.tail_len = kv.tail_len;
  P.k_codes = kv.k_codes;
  P.k_scale = static_cast<const uint16_t*>(kv.k_scale);
  P.k_zero = static_cast<const uint16_t*>(kv.k_zero);
  P.v_codes = kv.v_codes;
  P.v_scale = static_cast<const uint16_t*>(kv.v_scale);
  P.v_zero = static_cast<const uint16_t*>(kv.v_zero);
  P.kept_idx = kv.kept_idx;
  P.src_k = static_cast<const uint16_t*>(kv.src_k);
  P.src_v = static_cast<const uint16_t*>(kv.src_v);
  P.tail_k = static_cast<const uint16_t*>(kv.tail_k);
  P.tail_v = static_cast<const uint16_t*>(kv.tail_v);

  const dim3 grid(plan.splits, sh.n_kv_heads, sh.batch);
  const int D = sh.head_dim;
  if (kv.kind == VC_DRAFT_KIVI) {
    if (D == 128 && kv.bits == 2) launch_kivi<128, 2>(P, grid, stream);
    else if (D == 128 && kv.bits == 4) launch_kivi<128, 4>(P, grid, stream);
    else if (D == 64 && kv.bits == 2) launch_kivi<64, 2>(P, grid, stream);
    else launch_kivi<64, 4>(P, grid, stream);
  } else if (kv.kind == VC_DRAFT_TOKDROP) {
    if (D == 128) launch_rows<128, true>(P, grid, stream);
    else launch_rows<64, true>(P, grid, stream);
  } else {
    if (D == 128) launch_rows<128, false>(P, grid, stream);
    else launch_rows<64, false>(P, grid, stream);
  }
  vc_status st = check_launch("draft attention");
  if (st != VC_OK) return st;
  const dim3 mgrid(sh.n_q_heads, sh.batch);
  if (D == 128) hipLaunchKernelGGL((draft_merge_kernel<128>), mgrid, dim3(128), 0, stream, P);
  else hipLaunchKernelGGL((draft_merge_kernel<64>), mgrid, dim3(64), 0, stream, P);
  return check_launch("draft merge");
}

}  // namespace vc
