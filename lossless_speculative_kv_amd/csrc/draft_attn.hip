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
// MFMA mapping (v_mfma_f32_16x16x32; fp16 for KIVI and the fp16 tail, bf16
// for bf16 rows). NG = D/32 channel groups, HS = 16/NG query heads per head
// set, HPL = 4/NG heads per lane row.
//   QK: S[row][token] = sum_k A[row][k] B[k][token], B = the keys of 16
//       tokens, A = the query. Row (hl, j) = NG*hl + j pairs query head hl
//       with channel group j: in K-step kk the A row is nonzero only when
//       j == kk, so a lane folds the key scales of one 8-channel run only.
//       The result lane (q, t) holds rows 4q + r: every channel group of
//       HPL heads for token t. A full score is the sum of the lane's own
//       registers, and each lane owns distinct (head, token) scores, so the
//       softmax runs once per score.
//   P: a lane packs the probabilities of its tokens t and t + 16 into one
//       16-bit pair and hands them over through a small per-wave LDS area.
//   PV: O^T[channel][col] = sum_t V^T[channel][t] P~[t][col] with
//       P~[t][(hl, j)] = p[t][hl] * value_scale[t][group j]; output column
//       (hl, j) is kept only for channels of group j. Contraction slots 2r and
//       2r + 1 of lane group q are tokens 4q + r and 4q + r + 16.
//   The key scale and log2(e)/sqrt(D) are folded into the fp16 query per
//   32-token key group; key zero points give a per-(head, block) score
//   bias. Value zero points add sum_t p[t] * zero[t][j] per (head, j).
//
// Codes become fp16 MFMA operands through the gfx950 scaled narrow-float
// conversions, two per instruction: a 2-bit code in the two low bits of a
// nibble is the e2m1 value code/2, a 4-bit code in the low nibble of a byte
// is the e4m3 value code * 2^-9, so scales 2 and 2^9 give the code exactly.
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

template <int D>
struct Geo {
  static constexpr int NG = D / 32, HS = 16 / NG, HPL = 4 / NG, MT = D / 16, CPL = D / 16;
};

// ---------------------------------------------------------------- codes ----
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t m) {
  return as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, BYTE));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t m) {
  return as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 512.0f, HI));
}
// 2-bit word (code i at bits 2i) -> R[2b + k] = (code 4b + k, code 4b + 2 + k).
__device__ __forceinline__ void unpack2(uint32_t w, uint32_t (&R)[8]) {
  const uint32_t m0 = w & 0x33333333u, m1 = (w >> 2) & 0x33333333u;
  R[0] = fp4_pair<0>(m0);
  R[1] = fp4_pair<0>(m1);
  R[2] = fp4_pair<1>(m0);
  R[3] = fp4_pair<1>(m1);
  R[4] = fp4_pair<2>(m0);
  R[5] = fp4_pair<2>(m1);
  R[6] = fp4_pair<3>(m0);
  R[7] = fp4_pair<3>(m1);
}
// 4-bit word (code i at bits 4i) -> R[2h + k] = (code 4h + k, code 4h + 2 + k).
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t (&R)[4]) {
  const uint32_t m0 = w & 0x0F0F0F0Fu, m1 = (w >> 4) & 0x0F0F0F0Fu;
  R[0] = fp8_pair<false>(m0);
  R[1] = fp8_pair<false>(m1);
  R[2] = fp8_pair<true>(m0);
  R[3] = fp8_pair<true>(m1);
}
// Channel (within the lane's 8-channel key run) of contraction slot s: the
// unpacked pairs hold run channels (4(r>>1) + (r&1), that + 2) in register r.
__device__ __forceinline__ constexpr int kperm(int s) { return 4 * (s >> 2) + ((s >> 1) & 1) + 2 * (s & 1); }

// Key operand of tile i, K-step kk from the tile's raw words.
template <int BITS, int NWL>
__device__ __forceinline__ void key_operand(const uint32_t (&kw)[NWL], int kk, uint32_t (&B)[4]) {
  if constexpr (BITS == 2) {
    uint32_t R[8];
    unpack2(kw[kk >> 1], R);
#pragma unroll
    for (int r = 0; r < 4; ++r) B[r] = R[4 * (kk & 1) + r];
  } else {
    uint32_t R[4];
    unpack4(kw[kk], R);
#pragma unroll
    for (int r = 0; r < 4; ++r) B[r] = R[r];
  }
}
// Value operand of channel tile m (slots 2r, 2r + 1 of register r).
template <int BITS, int VWL>
__device__ __forceinline__ void value_operand(const uint32_t (&vw)[VWL], int m, uint32_t (&A)[4]) {
  if constexpr (BITS == 2) {
    uint32_t R[8];
    unpack2(vw[m >> 1], R);
#pragma unroll
    for (int r = 0; r < 4; ++r) A[r] = R[2 * r + (m & 1)];
  } else {
    uint32_t R[4];
    unpack4(vw[m], R);
#pragma unroll
    for (int r = 0; r < 4; ++r) A[r] = R[r];
  }
}

// ------------------------------------------------------ softmax state ----
// m, l: score layout (lane (q, t) owns heads HPL*q + u of each set);
// zt, acc: PV layout (lane n = (hl, j) owns output column (hl, j)).
template <int D, int NHS>
struct DState {
  static constexpr int HPL = Geo<D>::HPL, MT = Geo<D>::MT;
  float m[NHS][HPL];  // running max, uniform over the lane row
  float l[NHS][HPL];  // this lane's share of sum p
  float zt[NHS];      // this lane's share of sum p * value zero point (KIVI)
  f32x4 acc[NHS][MT];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < NHS; ++h) {
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
        m[h][u] = kNegInf;
        l[h][u] = 0.f;
      }
      zt[h] = 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Per-wave LDS area for the probability hand-over: [NHS][HS][16] words.
template <int D, int NHS>
constexpr int p_area_words() {
  return NHS * Geo<D>::HS * 16;
}

// Online softmax over one 32-token block of head set h and hand-over of the
// probabilities to the PV operand layout.
//   s[u][i]: score of head HPL*q + u, token 16i + t (log2 units, -inf for
//            invalid tokens), bias[u] added on top;
//   P[r]   : on return, the (token 4q' + r, token 4q' + r + 16) probability
//            pair of head hl(n) for this lane's PV column.
// The max only moves when a score exceeds it by more than kRescaleThreshold
// (so p <= 2^8), which makes the rescale of the accumulators rare; the
// result is the same softmax.
template <int D, int NHS, bool BF16>
__device__ __forceinline__ void soft_block(DState<D, NHS>& st, int h, const float (&s)[Geo<D>::HPL][2],
                                           const float (&bias)[Geo<D>::HPL], int lane, uint32_t* lds_p,
                                           uint32_t (&P)[4]) {
  constexpr int NG = Geo<D>::NG, HS = Geo<D>::HS, HPL = Geo<D>::HPL, MT = Geo<D>::MT;
  const int t = lane & 15, qg = lane >> 4, n = lane & 15, hl = n / NG;
  bool need = false;
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    const float lim = st.m[h][u] + kRescaleThreshold - bias[u];
    need = need || (s[u][0] > lim) || (s[u][1] > lim);
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    float alpha[HPL];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const float bm = row_max16(fmaxf(s[u][0], s[u][1]) + bias[u]);
      const bool up = bm > st.m[h][u] + kRescaleThreshold;
      alpha[u] = up ? fast_exp2(st.m[h][u] - bm) : 1.f;
      st.m[h][u] = up ? bm : st.m[h][u];
      st.l[h][u] *= alpha[u];
    }
    // the PV column (hl, j) takes the factor of head hl from lane row hl / HPL
    const int src = 4 * 16 * (hl / HPL);
    float a = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(alpha[0])));
    if constexpr (HPL == 2) {
      const float a1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(alpha[1])));
      a = (hl & 1) ? a1 : a;
    }
    st.zt[h] *= a;
#pragma unroll
    for (int m = 0; m < MT; ++m) st.acc[h][m] *= a;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    const float mb = st.m[h][u] - bias[u];
    const float p0 = fast_exp2(s[u][0] - mb), p1 = fast_exp2(s[u][1] - mb);
    st.l[h][u] += p0 + p1;
    lds_p[(h * HS + HPL * qg + u) * 16 + t] = pack16<BF16>(p0, p1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds_p + (h * HS + hl) * 16 + 4 * qg);
  P[0] = v[0];
  P[1] = v[1];
  P[2] = v[2];
  P[3] = v[3];
}

// Full scores of the lane's HPL heads from the NG partial rows.
template <int D>
__device__ __forceinline__ void row_scores(const f32x4 (&c)[2], float scale, float (&s)[Geo<D>::HPL][2]) {
  constexpr int NG = Geo<D>::NG, HPL = Geo<D>::HPL;
#pragma unroll
  for (int u = 0; u < HPL; ++u)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float x = c[i][NG * u];
#pragma unroll
      for (int jj = 1; jj < NG; ++jj) x += c[i][NG * u + jj];
      s[u][i] = x * scale;
    }
}

// ------------------------------------------------------- KIVI body block ----
// Buffer resources of one (sequence, KV head) unit; per-block offsets go in
// the scalar offset, so the loop does no vector address arithmetic. Loads
// past a unit's extent return zero.
struct KiviRes {
  __amdgpu_buffer_rsrc_t kc, ks, kz, vc, vs, vz;
};
constexpr int kRsrcWord3 = 0x00020000;

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const T* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, (int)bytes, kRsrcWord3);
}

template <int D, int BITS>
struct KiviRaw {
  static constexpr int NWL = D * BITS / 128, VWL = D * BITS / 64, CPL = Geo<D>::CPL;
  uint32_t kw[2][NWL];   // key codes of tokens t and t + 16
  uint32_t vw[VWL];      // value codes of the lane's slots
  uint32_t ks[4];        // key scales of the lane's 8-channel run
  uint32_t kz[CPL / 2];  // key zero points of channels CPL*t ..
  u32x4 vs, vz;          // value scales / zeros of the lane's 8 slots
};

template <int N>
__device__ __forceinline__ void buf_words(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = v[0];
    w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * i, soff, 0);
      w[i] = v[0];
      w[i + 1] = v[1];
      w[i + 2] = v[2];
      w[i + 3] = v[3];
    }
  }
}

// Lane-constant byte offsets into the unit's arrays.
struct KiviOffs {
  int kc0, kc1, ksc, kzc, vc, vsd;
};

template <int D, int BITS>
__device__ __forceinline__ KiviOffs kivi_offsets(int lane) {
  constexpr int NG = D / 32, WPT = D * BITS / 32, NWL = D * BITS / 128, VWL = D * BITS / 64, CPL = D / 16;
  const int n = lane & 15, qg = lane >> 4, j = n % NG;
  KiviOffs o;
  o.kc0 = (n * WPT + qg * NWL) * 4;
  o.kc1 = ((16 + n) * WPT + qg * NWL) * 4;
  o.ksc = 8 * (qg * NG + j) * 2;
  o.kzc = CPL * n * 2;
  o.vc = lane * VWL * 4;
  o.vsd = (j * 32 + qg * 8) * 2;
  return o;
}

template <int D, int BITS>
__device__ __forceinline__ void kivi_load(KiviRaw<D, BITS>& r, const KiviRes& res, const KiviOffs& o, int blk) {
  constexpr int NG = D / 32, WPT = D * BITS / 32, NWL = D * BITS / 128, VWL = D * BITS / 64, CPL = D / 16;
  // blk is wave-uniform; the scalar offsets must live in SGPRs
  blk = __builtin_amdgcn_readfirstlane(blk);
  const int skc = blk * 32 * WPT * 4, sks = blk * D * 2, svc = blk * 64 * VWL * 4, svs = blk * NG * 32 * 2;
  buf_words<NWL>(res.kc, o.kc0, skc, r.kw[0]);
  buf_words<NWL>(res.kc, o.kc1, skc, r.kw[1]);
  buf_words<VWL>(res.vc, o.vc, svc, r.vw);
  buf_words<4>(res.ks, o.ksc, sks, r.ks);
  buf_words<CPL / 2>(res.kz, o.kzc, sks, r.kz);
  uint32_t t[4];
  buf_words<4>(res.vs, o.vsd, svs, t);
  r.vs = u32x4{t[0], t[1], t[2], t[3]};
  buf_words<4>(res.vz, o.vsd, svs, t);
  r.vz = u32x4{t[0], t[1], t[2], t[3]};
}

// Query data of one wave, fixed over the body.
//   qf: PV/A layout, lane (q, (hl, j)): q[h*HS + hl][8(q*NG + j) + kperm(s)]
//       * log2(e)/sqrt(D), zero for padding heads;
//   qh, ql: score layout, lane (q, t): the same scaled query of head
//       h*HS + HPL*q + u at channels CPL*t + 2p, + 1, split into an fp16
//       pair and the fp16 pair of its remainder.
template <int D, int NHS>
struct KiviQuery {
  static constexpr int HPL = Geo<D>::HPL, CPL = Geo<D>::CPL;
  float qf[NHS][8];
  uint32_t qh[NHS][HPL][CPL / 2], ql[NHS][HPL][CPL / 2];
};

template <int D, int NHS>
__device__ __forceinline__ void kivi_query(const DraftParams& P, int b, int hk, int lane, KiviQuery<D, NHS>& Q) {
  constexpr int NG = Geo<D>::NG, HS = Geo<D>::HS, HPL = Geo<D>::HPL, CPL = Geo<D>::CPL;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
  const uint16_t* qb = P.q + ((size_t)b * P.Hq + (size_t)hk * P.g) * D;
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const int head = h * HS + hl;
    const bool ok = head < P.g;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      Q.qf[h][s] = ok ? bf16_bits_to_f32(qb[(size_t)head * D + 8 * (qg * NG + j) + kperm(s)]) * P.qscale : 0.f;
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const int hb = h * HS + HPL * qg + u;
      const bool okb = hb < P.g;
#pragma unroll
      for (int p = 0; p < CPL / 2; ++p) {
        float x[2], hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          x[e] = okb ? bf16_bits_to_f32(qb[(size_t)hb * D + CPL * n + 2 * p + e]) * P.qscale : 0.f;
          hi[e] = (float)(_Float16)x[e];
          lo[e] = x[e] - hi[e];
        }
        Q.qh[h][u][p] = pack_f16(hi[0], hi[1]);
        Q.ql[h][u][p] = pack_f16(lo[0], lo[1]);
      }
    }
  }
}

// One 32-token block of the quantised body.
template <int D, int BITS, int NHS>
__device__ __forceinline__ void kivi_compute(const KiviRaw<D, BITS>& raw, int lane, const KiviQuery<D, NHS>& Q,
                                             DState<D, NHS>& st, uint32_t* lds_p) {
  constexpr int NG = Geo<D>::NG, HPL = Geo<D>::HPL, MT = Geo<D>::MT, CPL = Geo<D>::CPL;
  constexpr int NWL = KiviRaw<D, BITS>::NWL, VWL = KiviRaw<D, BITS>::VWL;
  const int n = lane & 15, j = n % NG;

  // key operands of both token tiles, all K-steps
  uint32_t Bk[2][NG][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kk = 0; kk < NG; ++kk) key_operand<BITS, NWL>(raw.kw[i], kk, Bk[i][kk]);

  uint32_t vs[4], vz[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    vs[r] = raw.vs[r];
    vz[r] = raw.vz[r];
  }

  uint32_t Pv[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    // query with the key scales of this lane's run folded in (one rounding)
    uint32_t Aq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t w0 = raw.ks[2 * (r >> 1)], w1 = raw.ks[2 * (r >> 1) + 1];
      const float s0 = (r & 1) ? f16_hi(w0) : f16_lo(w0);
      const float s1 = (r & 1) ? f16_hi(w1) : f16_lo(w1);
      Aq[r] = pack_f16(Q.qf[h][2 * r] * s0, Q.qf[h][2 * r + 1] * s1);
    }
    // zero-point bias of the lane's heads: sum over channels CPL*t .. and the row
    float bias[HPL];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      float x = 0.f;
#pragma unroll
      for (int p = 0; p < CPL / 2; ++p) {
        x = __builtin_amdgcn_fdot2(as_f16x2(Q.qh[h][u][p]), as_f16x2(raw.kz[p]), x, false);
        x = __builtin_amdgcn_fdot2(as_f16x2(Q.ql[h][u][p]), as_f16x2(raw.kz[p]), x, false);
      }
      bias[u] = row_sum16(x);
    }
    f32x4 c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const bool on = (j == kk);
        const u32x4 a = {on ? Aq[0] : 0u, on ? Aq[1] : 0u, on ? Aq[2] : 0u, on ? Aq[3] : 0u};
        c[i] = mfma_f16(a, u32x4{Bk[i][kk][0], Bk[i][kk][1], Bk[i][kk][2], Bk[i][kk][3]}, c[i]);
      }
    }
    float s[HPL][2];
    row_scores<D>(c, 1.f, s);
    uint32_t Pp[4];
    soft_block<D, NHS, false>(st, h, s, bias, lane, lds_p, Pp);
    // value scales into P~, value zero points into zt
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t pr = Pp[r];
      st.zt[h] = __builtin_amdgcn_fdot2(as_f16x2(pr), as_f16x2(vz[r]), st.zt[h], false);
      Pv[h][r] = as_u32(as_f16x2(pr) * as_f16x2(vs[r]));
    }
  }

  // ---- PV ----
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
    value_operand<BITS, VWL>(raw.vw, m, A);
#pragma unroll
    for (int h = 0; h < NHS; ++h)
      st.acc[h][m] = mfma_f16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Pv[h][0], Pv[h][1], Pv[h][2], Pv[h][3]},
                              st.acc[h][m]);
  }
}

// ------------------------------------------------ unquantised row block ----
// A 32-token block of 16-bit rows (fp16 KIVI tail, or bf16 rows for token
// drop / dense). rows.k(t) / rows.v(t) give the row pointers of token
// t < nvalid. Aqm[h][kk] is the unscaled query operand of K-step kk (exact
// in fp16 and bf16, zero unless kk is the lane's group); scores are scaled
// by log2(e)/sqrt(D) after the MFMA.
// lds: this wave's staging area, 32 rows of D halfs with a stride of D + 4.
template <int D, int NHS, bool BF16, typename RowFn>
__device__ __forceinline__ void row_block(const RowFn& rows, int nvalid, int lane, float qscale,
                                          const uint32_t (&Aqm)[NHS][D / 32][4], DState<D, NHS>& st,
                                          uint16_t* lds, uint32_t* lds_p) {
  constexpr int NG = Geo<D>::NG, HPL = Geo<D>::HPL, MT = Geo<D>::MT, LSTR = D + 4;
  const int n = lane & 15, qg = lane >> 4;

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

  // ---- key operands: token 16i + n, channels 8(qg*NG + kk) .. + 7 ----
  uint32_t Bk[2][NG][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 16 * i + n;
    if (t < nvalid) {
      const uint16_t* kp = rows.k(t) + 8 * qg * NG;
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(kp + 8 * kk);
        Bk[i][kk][0] = v[0];
        Bk[i][kk][1] = v[1];
        Bk[i][kk][2] = v[2];
        Bk[i][kk][3] = v[3];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) Bk[i][kk][0] = Bk[i][kk][1] = Bk[i][kk][2] = Bk[i][kk][3] = 0u;
    }
  }

  uint32_t Pv[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    f32x4 c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk)
        c[i] = mfma16<BF16>(u32x4{Aqm[h][kk][0], Aqm[h][kk][1], Aqm[h][kk][2], Aqm[h][kk][3]},
                            u32x4{Bk[i][kk][0], Bk[i][kk][1], Bk[i][kk][2], Bk[i][kk][3]}, c[i]);
    }
    float s[HPL][2];
    row_scores<D>(c, qscale, s);
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      if (n >= nvalid) s[u][0] = kNegInf;
      if (16 + n >= nvalid) s[u][1] = kNegInf;
    }
    const float bias[HPL] = {};
    soft_block<D, NHS, BF16>(st, h, s, bias, lane, lds_p, Pv[h]);
  }

  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t lo = lds[(4 * qg + r) * LSTR + 16 * m + n];
      const uint32_t hi = lds[(16 + 4 * qg + r) * LSTR + 16 * m + n];
      A[r] = lo | (hi << 16);
    }
#pragma unroll
    for (int h = 0; h < NHS; ++h)
      st.acc[h][m] = mfma16<BF16>(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Pv[h][0], Pv[h][1], Pv[h][2], Pv[h][3]},
                                  st.acc[h][m]);
  }
}

// Unscaled query operands of the row path, one per K-step (zero unless the
// step is the lane's channel group).
template <int D, int NHS, bool BF16>
__device__ __forceinline__ void row_query(const DraftParams& P, int b, int hk, int lane,
                                          uint32_t (&Aqm)[NHS][D / 32][4]) {
  constexpr int NG = Geo<D>::NG, HS = Geo<D>::HS;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
  const uint16_t* qb = P.q + ((size_t)b * P.Hq + (size_t)hk * P.g) * D;
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const int head = h * HS + hl;
    const bool ok = head < P.g;
    uint32_t a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t* qp = qb + (size_t)(ok ? head : 0) * D + 8 * (qg * NG + j) + 2 * r;
      const float lo = ok ? bf16_bits_to_f32(qp[0]) : 0.f, hi = ok ? bf16_bits_to_f32(qp[1]) : 0.f;
      a[r] = pack16<BF16>(lo, hi);
    }
#pragma unroll
    for (int kk = 0; kk < NG; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) Aqm[h][kk][r] = (kk == j) ? a[r] : 0u;
  }
}

// Merge the 4 wave states of the workgroup and store the split's partial
// (running max, sum and unnormalised output per query head). lds must hold
// kWaves * NH * (D + 2) floats; it may alias the row staging area (the
// leading barrier orders the reuse). The splits are merged by a second
// kernel: a merge by the last workgroup to finish would need a device-scope
// release and acquire in every workgroup, which on a part whose L2 is split
// per XCD means an L2 writeback and invalidate each.
template <int D, int NHS>
__device__ __forceinline__ void store_partial(const DraftParams& P, int b, int hk, int split, int lane, int wave,
                                              DState<D, NHS>& st, bool has_zero, float* lds) {
  constexpr int NG = Geo<D>::NG, HS = Geo<D>::HS, HPL = Geo<D>::HPL, NH = NHS * HS;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
  float* lds_o = lds;
  float* lds_ml = lds + kWaves * NH * D;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const float zt = has_zero ? sum_q(st.zt[h]) : 0.f;
    const int head = h * HS + hl;
    float* o = lds_o + ((size_t)wave * NH + head) * D;
    // column (hl, j) is valid for the two channel tiles of group j. The tile
    // index is lane-dependent, so the values are picked with selects: an
    // indexed access (or branches the compiler folds into one) would move the
    // accumulators to scratch memory.
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = st.acc[h][mm][r];
#pragma unroll
        for (int jj = 1; jj < NG; ++jj) {
          const float w = st.acc[h][2 * jj + mm][r];
          v = (j == jj) ? w : v;
        }
        o[16 * (2 * j + mm) + 4 * qg + r] = v + zt;
      }
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const float l = row_sum16(st.l[h][u]);
      const int hb = h * HS + HPL * qg + u;
      if (n == 0) {
        lds_ml[(wave * NH + hb) * 2] = st.m[h][u];
        lds_ml[(wave * NH + hb) * 2 + 1] = l;
      }
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

// LDS: the row staging area (aliased by the wave merge), then the per-wave
// probability hand-over areas.
template <int D, int NHS>
constexpr size_t draft_stage_bytes() {
  constexpr int NH = NHS * Geo<D>::HS;
  constexpr size_t part = (size_t)kWaves * NH * (D + 2) * sizeof(float);
  constexpr size_t rows = (size_t)kWaves * 32 * (D + 4) * sizeof(uint16_t);
  return part > rows ? part : rows;
}
template <int D, int NHS>
constexpr size_t draft_lds_bytes() {
  return draft_stage_bytes<D, NHS>() + (size_t)kWaves * p_area_words<D, NHS>() * sizeof(uint32_t);
}

// ---------------------------------------------------------------- kernels ----
template <int D, int BITS, int NHS>
__global__ __launch_bounds__(256) void draft_kivi_kernel(const DraftParams P) {
  constexpr int NG = Geo<D>::NG, WPT = D * BITS / 32, VWL = D * BITS / 64;
  __shared__ __attribute__((aligned(16))) char smem[draft_lds_bytes<D, NHS>()];
  // the wave index is uniform across the wave; saying so keeps the per-block
  // buffer offsets in SGPRs (no waterfall loops around the loads)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  uint32_t* lds_p = reinterpret_cast<uint32_t*>(smem + draft_stage_bytes<D, NHS>()) + wave * p_area_words<D, NHS>();

  DState<D, NHS> st;
  st.init();
  const bool tail_split = (split == P.S - 1);
  if (!tail_split) {
    KiviQuery<D, NHS> Q;
    kivi_query<D, NHS>(P, b, hk, lane, Q);
    const int nblk = min(max(P.body_len[b], 0), P.body_cap) / 32;
    const int b0 = (split * kWaves + wave) * P.bpw;
    const int b1 = min(b0 + P.bpw, nblk);
    if (b0 < b1) {
      const size_t nbc = (size_t)(P.body_cap / 32);
      KiviRes res;
      res.kc = make_rsrc(P.k_codes + unit * P.body_cap * WPT, (size_t)P.body_cap * WPT * 4);
      res.ks = make_rsrc(P.k_scale + unit * nbc * D, nbc * D * 2);
      res.kz = make_rsrc(P.k_zero + unit * nbc * D, nbc * D * 2);
      res.vc = make_rsrc(P.v_codes + unit * nbc * 64 * VWL, nbc * 64 * VWL * 4);
      res.vs = make_rsrc(P.v_scale + unit * nbc * NG * 32, nbc * NG * 32 * 2);
      res.vz = make_rsrc(P.v_zero + unit * nbc * NG * 32, nbc * NG * 32 * 2);
      const KiviOffs offs = kivi_offsets<D, BITS>(lane);
      // two register sets in ping-pong: the loads of block i+1 are in flight
      // while block i is computed. The loads are unconditional (the index is
      // clamped to the wave's last block, a cache hit) so that no register
      // copy has to wait for a load that was just issued.
      const int last = b1 - 1;
      KiviRaw<D, BITS> ra, rb;
      kivi_load<D, BITS>(ra, res, offs, b0);
      for (int blk = b0;; blk += 2) {
        kivi_load<D, BITS>(rb, res, offs, min(blk + 1, last));
        kivi_compute<D, BITS, NHS>(ra, lane, Q, st, lds_p);
        if (blk + 1 > last) break;
        kivi_load<D, BITS>(ra, res, offs, min(blk + 2, last));
        kivi_compute<D, BITS, NHS>(rb, lane, Q, st, lds_p);
        if (blk + 2 > last) break;
      }
    }
  } else {
    uint32_t Aqm[NHS][D / 32][4];
    row_query<D, NHS, false>(P, b, hk, lane, Aqm);
    const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
    const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
    const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
    uint16_t* my_lds = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 4);
    for (int blk = wave; blk * 32 < nt; blk += kWaves) {
      const PlainRows<D> rows{tk + (size_t)blk * 32 * D, tv + (size_t)blk * 32 * D};
      row_block<D, NHS, false>(rows, min(32, nt - blk * 32), lane, P.qscale, Aqm, st, my_lds, lds_p);
    }
  }
  store_partial<D, NHS>(P, b, hk, split, lane, wave, st, !tail_split, reinterpret_cast<float*>(smem));
}

// Token-drop (GATHER) and dense draft caches: bf16 rows everywhere.
template <int D, int NHS, bool GATHER>
__global__ __launch_bounds__(256) void draft_rows_kernel(const DraftParams P) {
  __shared__ __attribute__((aligned(16))) char smem[draft_lds_bytes<D, NHS>()];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  uint32_t* lds_p = reinterpret_cast<uint32_t*>(smem + draft_stage_bytes<D, NHS>()) + wave * p_area_words<D, NHS>();

  DState<D, NHS> st;
  st.init();
  uint32_t Aqm[NHS][D / 32][4];
  row_query<D, NHS, true>(P, b, hk, lane, Aqm);
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
      row_block<D, NHS, true>(rows, min(32, nb - blk * 32), lane, P.qscale, Aqm, st, my_lds, lds_p);
    }
  } else {
    const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
    const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
    const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
    for (int blk = wave; blk * 32 < nt; blk += kWaves) {
      const PlainRows<D> rows{tk + (size_t)blk * 32 * D, tv + (size_t)blk * 32 * D};
      row_block<D, NHS, true>(rows, min(32, nt - blk * 32), lane, P.qscale, Aqm, st, my_lds, lds_p);
    }
  }
  store_partial<D, NHS>(P, b, hk, split, lane, wave, st, false, reinterpret_cast<float*>(smem));
}

// Merge the splits of one (sequence, query head) in split order, so the
// result does not depend on the order in which workgroups ran.
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

// Workspace: the split partials (unnormalised outputs, then max and sum).
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
  char* w = static_cast<char*>(ws);
  P.part_o = reinterpret_cast<float*>(w);
  w += align_up(rows * sh.head_dim * sizeof(float), 256);
  P.part_ml = reinterpret_cast<float*>(w);
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
