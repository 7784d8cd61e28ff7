// Draft decode attention over the compressed cache (VeriCache summary, "Core
// algorithm": drafting runs the target model over KV_comp; "P1": drafting is
// bound by HBM bandwidth, so the kernel streams the compressed bytes once and
// dequantises in registers).
//
// Work decomposition: one workgroup per (split, KV head, sequence). A KIVI
// workgroup has NW body waves, which are dealt the split's quantised 32-token
// blocks in turn, and one wave for the split's share of the fp16 tail; a row
// workgroup (token drop, dense) has as many waves as its registers allow on a
// CU, dealt the split's blocks in turn, each then taking a share of the tail.
// Every workgroup fills its CU, and waves that share a SIMD are paced (see
// pace_waves). Every wave keeps an online-softmax state for all g query heads
// of the KV head; the wave states are merged through LDS into a per-split
// partial (max, sum, unnormalised output), and the last workgroup of a
// (KV head, sequence) to store its partial merges the partials in a fixed
// order (split groups of up to 16 splits, each in split order, then the
// groups in order).
//
// MFMA mapping (v_mfma_f32_16x16x32; fp16 for KIVI and the fp16 tail, bf16
// for the scores of bf16 rows, fp16 for every P x V: probabilities in fp16,
// bf16 value rows converted exactly). NG = D/32 channel groups, W groups per MFMA row, NR = NG/W
// row groups per head, HS = 16/NR query heads per head set, HPL = 4/NR heads
// per lane row. The KIVI kernel takes the narrowest W with HS >= g (one head
// set); the row kernel uses W = 1 and several head sets when g > HS.
//   QK: S[row][token] = sum_k A[row][k] B[k][token], B = the keys of 16
//       tokens, A = the query. Row (hl, jr) = NR*hl + jr pairs query head hl
//       with row group jr: in K-step kk the A row is nonzero only when
//       kk / W == jr, so a lane folds the key scales of W 8-channel runs
//       only. The result lane (q, t) holds rows 4q + r: every row group of
//       HPL heads for token t. A full score is the sum of the lane's own
//       registers, and each lane owns distinct (head, token) scores, so the
//       softmax runs once per score.
//   P: a lane packs the probabilities of its tokens t and t + 16 into one
//       16-bit pair and hands them over through a small per-wave LDS area.
//   PV: O^T[channel][col] = sum_t V^T[channel][t] P~[t][col] with
//       P~[t][(hl, jr)] = p[t][hl] * value_scale[t][group of the channel
//       tile] (one P~ per group of the row group); output column (hl, jr) is
//       kept only for channels of row group jr. Contraction slots 2r and
//       2r + 1 of lane group q are tokens 4q + r and 4q + r + 16.
//   The key scale and log2(e)/sqrt(D) are folded into the fp16 query per
//   32-token key group; key zero points give a per-(head, block) score
//   bias. Value zero points add sum_t p[t] * zero[t][j] per (head, j).
//
// Codes become fp16 MFMA operands through the gfx950 scaled narrow-float
// conversions, two per instruction: a 2-bit code in the two low bits of a
// nibble is the e2m1 value code/2, a 4-bit code in the low nibble of a byte
// is the e4m3 value code * 2^-9, so scales 2 and 2^9 give the code exactly.
#include <map>
#include <mutex>

#include "attn_common.h"

namespace vc {

namespace {


struct DraftParams {
  const uint16_t* q;  // bf16 [B][Hq][D]
  float* part_o;      // [B][Hq][S][D]
  float* part_ml;     // [B][Hq][S][2]
  float* out;         // [B][Hq][D]
  uint32_t* counters;  // [B][Hkv] splits stored so far (zero between calls)
  int B, Hq, Hkv, g, S, bpw;
  float qscale;       // log2(e) / sqrt(D)
  int body_cap, tail_cap, src_t_cap;
  const int32_t* body_len;
  const int32_t* tail_len;
  const char* kivi_blocks;  // KIVI body records [u][body_cap/32][BlockLayout::BYTES]
  const int32_t* kept_idx;
  const uint16_t* src_k;
  const uint16_t* src_v;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
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

// ------------------------------------------------------ head geometry ----
// W channel groups per MFMA row: NR = NG/W row groups per head, HS = 16/NR
// query heads per head set, HPL = 4/NR heads per lane row of the score
// layout, MT = D/16 output channel tiles, CPL = D/16 key channels per lane
// for the zero-point bias.
template <int D, int W>
struct Geo {
  static constexpr int NG = D / 32, NR = NG / W, HS = 16 / NR, HPL = 4 / NR, MT = D / 16, CPL = D / 16;
  static_assert(W >= 1 && NG % W == 0, "row width");
};

// ------------------------------------------------------ softmax state ----
// m, l: score layout (lane (q, t) owns heads HPL*q + u of each set);
// zc, acc: PV layout (lane n = (hl, jr) owns output column (hl, jr)).
template <int D, int W, int NHS>
struct DState {
  static constexpr int HPL = Geo<D, W>::HPL, MT = Geo<D, W>::MT;
  float m[NHS][HPL];  // running max, uniform over the lane row
  float l[NHS][HPL];  // this lane's share of sum p
  f32x4 zc[NHS];      // KIVI: sum p * value zero point, MFMA layout: row g = channel group, column (hl, jr)
  f32x4 acc[NHS][MT];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < NHS; ++h) {
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
        m[h][u] = kNegInf;
        l[h][u] = 0.f;
      }
      zc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Per-wave LDS area for the probability hand-over: [NHS][HS][16] words.
template <int D, int W, int NHS>
constexpr int p_area_words() {
  return NHS * Geo<D, W>::HS * 16;
}

// Online softmax over one 32-token block of head set h and hand-over of the
// probabilities, rounded to fp16 (11 significant bits), to the PV operand
// layout.
//   s[u][i]: score of head HPL*q + u, token 16i + t (log2 units, -inf for
//            invalid tokens), bias[u] added on top;
//   P[r]   : on return, the (token 4q' + r, token 4q' + r + 16) probability
//            pair of head hl(n) for this lane's PV column.
// The max only moves when a score exceeds it by more than kRescaleThreshold
// (so p <= 2^8), which makes the rescale of the accumulators rare; the
// result is the same softmax.
template <int D, int W, int NHS>
__device__ __forceinline__ void soft_block(DState<D, W, NHS>& st, int h, const float (&s)[Geo<D, W>::HPL][2],
                                           const float (&bias)[Geo<D, W>::HPL], int lane, uint32_t* lds_p,
                                           uint32_t (&P)[4]) {
  using G = Geo<D, W>;
  constexpr int NR = G::NR, HS = G::HS, HPL = G::HPL, MT = G::MT;
  const int t = lane & 15, qg = lane >> 4, n = lane & 15, hl = n / NR;
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
    // the PV column (hl, jr) takes the factor of head hl from lane row hl / HPL
    const int src = 4 * 16 * (hl / HPL);
    float a = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(alpha[0])));
#pragma unroll
    for (int u = 1; u < HPL; ++u) {
      const float au = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(alpha[u])));
      a = (hl % HPL == u) ? au : a;
    }
    st.zc[h] *= a;
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
    lds_p[(h * HS + HPL * qg + u) * 16 + t] = pack_f16(p0, p1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds_p + (h * HS + hl) * 16 + 4 * qg);
  P[0] = v[0];
  P[1] = v[1];
  P[2] = v[2];
  P[3] = v[3];
}

// Full scores of the lane's HPL heads from the NR partial rows.
template <int D, int W>
__device__ __forceinline__ void row_scores(const f32x4 (&c)[2], float scale, float (&s)[Geo<D, W>::HPL][2]) {
  constexpr int NR = Geo<D, W>::NR, HPL = Geo<D, W>::HPL;
#pragma unroll
  for (int u = 0; u < HPL; ++u)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float x = c[i][NR * u];
#pragma unroll
      for (int jj = 1; jj < NR; ++jj) x += c[i][NR * u + jj];
      s[u][i] = x * scale;
    }
}

// ------------------------------------------------------- KIVI body block ----
// Each wave streams its own 32-token blocks into a private LDS ring with
// direct-to-LDS buffer loads issued ahead, then reads its operands from LDS.
// A block's record in memory has the same layout as its ring stage, so one
// block is one contiguous copy (1 KB per load instruction where it can).
template <int D, int BITS>
struct BlockLayout {
  static constexpr int NG = D / 32, WPT = D * BITS / 32, VWL = D * BITS / 64;
  static constexpr int KC = 0, KC_B = 32 * WPT * 4;        // key codes, token-major
  static constexpr int VC = KC + KC_B, VC_B = 64 * VWL * 4; // value codes, lane-major
  static constexpr int KS = VC + VC_B, KS_B = D * 2;        // key scales / zeros
  static constexpr int KZ = KS + KS_B;
  static constexpr int VS = KZ + KS_B, VS_B = NG * 32 * 2;  // value scales / zeros
  static constexpr int VZ = VS + VS_B;
  static constexpr int BYTES = VZ + VS_B;
  static_assert(BYTES == 8 * D * (BITS + 1), "record size");
  // direct-to-LDS instructions per block: 1 KB (16 B per lane), then 256 B
  // (4 B per lane), then a 128 B rest (4 B for half the lanes)
  static constexpr int pieces(int b) { return b / 1024 + (b % 1024) / 256 + ((b % 256) ? 1 : 0); }
  static constexpr int NI = pieces(BYTES);
  static_assert(KC_B % 128 == 0 && VC_B % 128 == 0 && KS_B % 128 == 0 && VS_B % 128 == 0, "128-byte pieces");
};

// s_waitcnt on the vector-memory counter only: vmcnt(N), others untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copy BYTES from global byte offset soff of r to dst (wave-uniform).
template <int BYTES>
__device__ __forceinline__ void dma_piece(__amdgpu_buffer_rsrc_t r, char* dst, int soff, int lane) {
  constexpr int N1K = BYTES / 1024, N256 = (BYTES % 1024) / 256, R128 = BYTES % 256;
#pragma unroll
  for (int i = 0; i < N1K; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, lane * 16, soff + i * 1024, 0,
                                             kStreamPolicy);
#pragma unroll
  for (int i = 0; i < N256; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + N1K * 1024 + i * 256), 4, lane * 4,
                                             soff + N1K * 1024 + i * 256, 0, kStreamPolicy);
  if constexpr (R128 != 0) {
    if (lane < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + N1K * 1024 + N256 * 256), 4, lane * 4,
                                               soff + N1K * 1024 + N256 * 256, 0, kStreamPolicy);
  }
}

// The unit's six arrays.
struct KiviRes {
  __amdgpu_buffer_rsrc_t blocks;  // the unit's block records
};

template <int D, int BITS>
__device__ __forceinline__ void issue_block(char* dst, const KiviRes& res, int blk, int lane) {
  using BL = BlockLayout<D, BITS>;
  blk = __builtin_amdgcn_readfirstlane(blk);
  dma_piece<BL::BYTES>(res.blocks, dst, blk * BL::BYTES, lane);
}

template <int N>
__device__ __forceinline__ void lds_words(const char* p, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0];
    w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + 4 * i);
      w[i] = v[0];
      w[i + 1] = v[1];
      w[i + 2] = v[2];
      w[i + 3] = v[3];
    }
  }
}

template <int D, int BITS, int W>
struct KiviRaw {
  static constexpr int NWL = D * BITS / 128, VWL = D * BITS / 64;
  uint32_t kw[2][NWL];  // key codes of tokens t and t + 16
  uint32_t vw[VWL];     // value codes of the lane's slots
  uint32_t ks[4 * W];   // key scales of the lane's W 8-channel runs
  u32x4 vs[W];          // value scales of the lane's 8 slots, per group
  u32x4 vz;             // value zeros of group n (lane n < NG) for the lane's 8 slots
};

// The lane's operands of one staged block.
template <int D, int BITS, int W>
__device__ __forceinline__ void kivi_read(KiviRaw<D, BITS, W>& r, const char* blk, int lane) {
  using BL = BlockLayout<D, BITS>;
  constexpr int NG = D / 32, NR = NG / W, WPT = BL::WPT, NWL = KiviRaw<D, BITS, W>::NWL, VWL = BL::VWL;
  const int n = lane & 15, qg = lane >> 4, jr = n % NR;
  lds_words<NWL>(blk + BL::KC + (n * WPT + qg * NWL) * 4, r.kw[0]);
  lds_words<NWL>(blk + BL::KC + ((16 + n) * WPT + qg * NWL) * 4, r.kw[1]);
  lds_words<VWL>(blk + BL::VC + lane * VWL * 4, r.vw);
  lds_words<4 * W>(blk + BL::KS + (qg * NG + W * jr) * 16, r.ks);
#pragma unroll
  for (int w = 0; w < W; ++w) {
    uint32_t t[4];
    lds_words<4>(blk + BL::VS + ((W * jr + w) * 32 + qg * 8) * 2, t);
    r.vs[w] = u32x4{t[0], t[1], t[2], t[3]};
  }
  {
    // rows of the zero-point product past the groups read group NG - 1
    // again; their results are never used
    uint32_t t[4];
    lds_words<4>(blk + BL::VZ + (min(n, NG - 1) * 32 + qg * 8) * 2, t);
    r.vz = u32x4{t[0], t[1], t[2], t[3]};
  }
}

// Query data of one wave, fixed over the body (one head set, g <= HS).
//   qm: A layout, lane (q, (hl, jr)), K-step kk (channel run q*NG + kk):
//       fp16 pairs (slots 2r, 2r + 1) of q[hl][8(q*NG + kk) + kperm(s)] when
//       kk / W == jr, zero otherwise and for padding heads (the scores are
//       scaled after the MFMA). Times the key scales it is the operand of
//       the codes; as it is, that of the key zero points, so row (hl, jr)
//       of the zero-point product holds the term of the channels of row
//       group jr, and the NR partial rows of a head add up as the scores do.
template <int D, int W>
struct KiviQuery {
  static constexpr int NG = Geo<D, W>::NG;
  uint32_t qm[NG][4];
  float qscale;  // log2(e)/sqrt(D), applied to the fp32 scores
};

// Raw bf16 bits of the query values a lane needs (pairs per word, lowest
// channel in the low half), loaded as whole 16-byte runs from a valid head
// (head 0 stands in for padding heads, whose values are zeroed on
// conversion). Unconditional vector loads leave the wave with one trip to
// memory; loads under a per-lane condition are issued and waited for one by
// one.
template <int D, int W>
struct KiviQueryRaw {
  uint32_t qp[W][4];  // channels 8(q*NG + W*jr + w) + 0..7 of head hl
};

template <int N>
__device__ __forceinline__ void global_words(const uint16_t* p, uint32_t* w) {
  if constexpr (N == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0];
    w[1] = v[1];
  } else {
    static_assert(N == 4, "16-byte runs");
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
}

__device__ __forceinline__ uint32_t half_of(const uint32_t* w, int i) { return (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu; }

template <int D, int W>
__device__ __forceinline__ void kivi_query_load(const DraftParams& P, int b, int hk, int lane, KiviQueryRaw<D, W>& R) {
  using G = Geo<D, W>;
  constexpr int NG = G::NG, NR = G::NR;
  const int n = lane & 15, qg = lane >> 4, jr = n % NR, hl = n / NR;
  const uint16_t* qb = P.q + ((size_t)b * P.Hq + (size_t)hk * P.g) * D;
  const int hlc = hl < P.g ? hl : 0;
#pragma unroll
  for (int w = 0; w < W; ++w) global_words<4>(qb + (size_t)hlc * D + 8 * (qg * NG + W * jr + w), R.qp[w]);
}

template <int D, int W>
__device__ __forceinline__ void kivi_query_finish(const DraftParams& P, int lane, const KiviQueryRaw<D, W>& R,
                                                  KiviQuery<D, W>& Q) {
  using G = Geo<D, W>;
  constexpr int NR = G::NR;
  const int n = lane & 15, hl = n / NR, jr = n % NR;
  const bool ok = hl < P.g;
#pragma unroll
  for (int kk = 0; kk < G::NG; ++kk) {
    const bool on = ok && jr == kk / W;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) x[e] = on ? bf16_bits_to_f32(half_of(R.qp[kk % W], kperm(2 * r + e))) : 0.f;
      // unscaled: a bf16 query value is an fp16 value (above 2^-14), so the
      // only rounding left before the MFMA is that of q * key scale
      Q.qm[kk][r] = pack_f16(x[0], x[1]);
    }
  }
  Q.qscale = P.qscale;
}

// One 32-token block of the quantised body.
// The key zero-point term sum_c q_c zero_c of each head on the MFMA: the
// unscaled query operand of each K-step times the zero points of its
// channel runs (stored in the runs' slot order), read from the block's ring
// stage; every token column gets the same term. The product is exact in
// fp32 and seeds both score tiles of kivi_compute.
template <int D, int BITS, int W>
__device__ __forceinline__ f32x4 kivi_zero_term(const char* stage, int lane, const KiviQuery<D, W>& Q) {
  using BL = BlockLayout<D, BITS>;
  constexpr int NG = D / 32;
  const int qg = lane >> 4;
  f32x4 cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NG; ++kk) {
    const u32x4 z = *reinterpret_cast<const u32x4*>(stage + BL::KZ + (qg * NG + kk) * 16);
    cb = mfma_f16(u32x4{Q.qm[kk][0], Q.qm[kk][1], Q.qm[kk][2], Q.qm[kk][3]}, z, cb);
  }
  return cb;
}

// cb: the key zero-point term from kivi_zero_term.
template <int D, int BITS, int W>
__device__ __forceinline__ void kivi_compute(const KiviRaw<D, BITS, W>& raw, const f32x4& cb, int lane,
                                             const KiviQuery<D, W>& Q, DState<D, W, 1>& st, uint32_t* lds_p) {
  using G = Geo<D, W>;
  constexpr int NG = G::NG, HPL = G::HPL, MT = G::MT;
  constexpr int NWL = KiviRaw<D, BITS, W>::NWL, VWL = KiviRaw<D, BITS, W>::VWL;

  // key operands of both token tiles, all K-steps
  uint32_t Bk[2][NG][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kk = 0; kk < NG; ++kk) key_operand<BITS, NWL>(raw.kw[i], kk, Bk[i][kk]);

  // query with the key scales of this lane's runs folded in: register r of
  // K-step kk pairs run channels kperm(2r), kperm(2r + 1), which is scale
  // word r of the run as stored; the lane's run of K-step kk is its run
  // kk mod W (K-steps of other row groups multiply a zero query). The
  // products are exact: a key scale has at most three significant bits and
  // a bf16 query value eight, within fp16's eleven.
  uint32_t Aq[NG][4];
#pragma unroll
  for (int kk = 0; kk < NG; ++kk)
#pragma unroll
    for (int r = 0; r < 4; ++r) Aq[kk][r] = as_u32(as_f16x2(Q.qm[kk][r]) * as_f16x2(raw.ks[4 * (kk % W) + r]));
  // the key zero-point term (cb) is already inside the scores
  float bias[HPL];
#pragma unroll
  for (int u = 0; u < HPL; ++u) bias[u] = 0.f;
  f32x4 c[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    c[i] = cb;
#pragma unroll
    for (int kk = 0; kk < NG; ++kk)
      c[i] = mfma_f16(u32x4{Aq[kk][0], Aq[kk][1], Aq[kk][2], Aq[kk][3]},
                      u32x4{Bk[i][kk][0], Bk[i][kk][1], Bk[i][kk][2], Bk[i][kk][3]}, c[i]);
  }
  float s[HPL][2];
  row_scores<D, W>(c, Q.qscale, s);
  uint32_t Pp[4];
  soft_block<D, W, 1>(st, 0, s, bias, lane, lds_p, Pp);
  // value scales into P~ (one per channel group of the column); the value
  // zero points on the MFMA: row g of zc gains sum_t zero[t][g] p[t] for
  // every column, with the same fp16 probabilities as the products
  uint32_t Pv[W][4];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) Pv[w][r] = as_u32(as_f16x2(Pp[r]) * as_f16x2(raw.vs[w][r]));
  st.zc[0] = mfma_f16(raw.vz, u32x4{Pp[0], Pp[1], Pp[2], Pp[3]}, st.zc[0]);

  // ---- PV: channel tile m belongs to group m/2, i.e. run (m/2) % W of the column ----
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
    value_operand<BITS, VWL>(raw.vw, m, A);
    const uint32_t* pv = Pv[(m >> 1) % W];
    st.acc[0][m] = mfma_f16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{pv[0], pv[1], pv[2], pv[3]}, st.acc[0][m]);
  }
}

// ------------------------------------------------ unquantised row block ----
// A 32-token block of 16-bit rows (fp16 KIVI tail, or bf16 rows for token
// drop / dense), W = 1 rows. rows.k(t, i) / rows.v(t, u) give the row
// pointers of token t < nvalid, which is key row 16i + n or value row
// lane / (D/8) + (512/D) u of the lane. Aqm[h][kk] is the unscaled query operand of K-step kk
// (exact in fp16 and bf16, zero unless kk is the lane's group); scores are
// scaled by log2(e)/sqrt(D) after the MFMA.
// lds: this wave's staging area for the value rows, 32 rows of D halfs with
// a stride of D + 4 (so a block takes one trip to memory: keys and values
// are loaded together, the V^T operand is then read from LDS). Values are
// staged in fp16 (bf16 rows converted on the way), so P x V runs on the f16
// MFMA with fp16 probabilities.
template <int D, int W, int NHS, bool BF16, typename RowFn>
__device__ __forceinline__ void row_block(const RowFn& rows, int nvalid, int lane, float qscale,
                                          const uint32_t (&Aqm)[NHS][D / 32][4], DState<D, W, NHS>& st,
                                          uint16_t* lds, uint32_t* lds_p) {
  using G = Geo<D, W>;
  constexpr int NG = G::NG, HPL = G::HPL, MT = G::MT, LSTR = D + 4;
  const int n = lane & 15, qg = lane >> 4;

  // ---- stage V rows in LDS (invalid rows as zeros) ----
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
      // every lane loads (a row past the block's end reads its last row and
      // is zeroed): a load under a per-lane condition waits on its own
      const int t = lane / CPR + RPI * u, c = lane % CPR;
      u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows.v(min(t, nvalid - 1), u) + 8 * c));
      if (t >= nvalid) v = u32x4{0u, 0u, 0u, 0u};
      if constexpr (BF16) {
        // bf16 values to fp16 for the fp16 probabilities' product: exact
        // for magnitudes 2^-17 .. 65504 (smaller ones round to 2^-24 steps)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_f16(__uint_as_float(v[e] << 16), __uint_as_float(v[e] & 0xFFFF0000u));
      }
      uint32_t* d = reinterpret_cast<uint32_t*>(lds + t * LSTR + 8 * c);
      *reinterpret_cast<u32x2*>(d) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(d + 2) = u32x2{v[2], v[3]};
    }
  }

  // ---- key operands: token 16i + n, channels 32kk + 8qg .. + 7 ----
  uint32_t Bk[2][NG][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 16 * i + n;
    const uint16_t* kp = rows.k(min(t, nvalid - 1), i) + 8 * qg;
    const bool ok = t < nvalid;
#pragma unroll
    for (int kk = 0; kk < NG; ++kk) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 32 * kk));
      Bk[i][kk][0] = ok ? v[0] : 0u;
      Bk[i][kk][1] = ok ? v[1] : 0u;
      Bk[i][kk][2] = ok ? v[2] : 0u;
      Bk[i][kk][3] = ok ? v[3] : 0u;
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
    row_scores<D, W>(c, qscale, s);
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      if (n >= nvalid) s[u][0] = kNegInf;
      if (16 + n >= nvalid) s[u][1] = kNegInf;
    }
    const float bias[HPL] = {};
    soft_block<D, W, NHS>(st, h, s, bias, lane, lds_p, Pv[h]);
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
      st.acc[h][m] = mfma_f16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Pv[h][0], Pv[h][1], Pv[h][2], Pv[h][3]},
                              st.acc[h][m]);
  }
}

// Unscaled query operands of the row path (W = 1), one per K-step (zero
// unless the step is the lane's channel group). K-step kk covers channels
// 32kk .. 32kk + 31, lane group qg the eight from 32kk + 8qg, so a key load
// instruction reads 64 contiguous bytes of each of 16 rows.
template <int D, int NHS, bool BF16>
__device__ __forceinline__ void row_query(const DraftParams& P, int b, int hk, int lane,
                                          uint32_t (&Aqm)[NHS][D / 32][4]) {
  constexpr int NG = Geo<D, 1>::NG, HS = Geo<D, 1>::HS;
  const int n = lane & 15, qg = lane >> 4, j = n % NG, hl = n / NG;
  const uint16_t* qb = P.q + ((size_t)b * P.Hq + (size_t)hk * P.g) * D;
  // every head set's run is loaded before any is used (one trip to memory);
  // padding heads read head 0 and are zeroed below
  uint32_t raw[NHS][4];
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const int head = h * HS + hl;
    global_words<4>(qb + (size_t)(head < P.g ? head : 0) * D + 32 * j + 8 * qg, raw[h]);
  }
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    const bool ok = h * HS + hl < P.g;
    uint32_t a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = ok ? bf16_bits_to_f32(raw[h][r] & 0xFFFFu) : 0.f;
      const float hi = ok ? bf16_bits_to_f32(raw[h][r] >> 16) : 0.f;
      a[r] = pack16<BF16>(lo, hi);
    }
#pragma unroll
    for (int kk = 0; kk < NG; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) Aqm[h][kk][r] = (kk == j) ? a[r] : 0u;
  }
}

// The value zero-point terms of this lane's PV column (hl, jr) for the
// channel tiles 2W jr + mm: row g = W jr + mm / 2 of zc, which lane n of
// lane group 0 holds (MFMA output rows 0..3).
template <int D, int W, int NHS>
__device__ __forceinline__ void zero_terms(const DState<D, W, NHS>& st, int h, int lane, float (&zt)[2 * W]) {
  using G = Geo<D, W>;
  const int n = lane & 15, jr = n % G::NR;
  float z[G::NG];
#pragma unroll
  for (int g = 0; g < G::NG; ++g)
    z[g] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * n, __float_as_int(st.zc[h][g])));
#pragma unroll
  for (int mm = 0; mm < 2 * W; ++mm) {
    float v = z[mm >> 1];
#pragma unroll
    for (int jj = 1; jj < G::NR; ++jj) v = (jr == jj) ? z[W * jj + (mm >> 1)] : v;
    zt[mm] = v;
  }
}

// The wave merge at the end of a workgroup. Each wave first writes its state
// in one layout for every state type: per query head of the unit, the
// unnormalised output row (D floats, the value zero-point term added) and
// (running max, sum). Then all threads merge the waves and store the split's
// partial, with device-coherent stores (they pass the per-XCD L2s), so the
// workgroup that merges the splits (finish_unit) reads them without an L2
// writeback or invalidate.
//   o: [NH][D] floats of this wave; ml: [NH][2] floats of this wave.
template <int D, int W, int NHS>
__device__ __forceinline__ void dump_state(int lane, DState<D, W, NHS>& st, bool has_zero, float* o, float* ml) {
  using G = Geo<D, W>;
  constexpr int NR = G::NR, HS = G::HS, HPL = G::HPL;
  const int n = lane & 15, qg = lane >> 4, jr = n % NR, hl = n / NR;
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    float* oh = o + (size_t)(h * HS + hl) * D;
    float ztm[2 * W] = {};
    if (has_zero) zero_terms<D, W, NHS>(st, h, lane, ztm);
    // column (hl, jr) is valid for the 2W channel tiles of row group jr. The
    // tile index is lane-dependent, so the values are picked with selects:
    // an indexed access (or branches the compiler folds into one) would move
    // the accumulators to scratch memory.
#pragma unroll
    for (int mm = 0; mm < 2 * W; ++mm) {
      const float zt = ztm[mm];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = st.acc[h][mm][r];
#pragma unroll
        for (int jj = 1; jj < NR; ++jj) {
          const float x = st.acc[h][2 * W * jj + mm][r];
          v = (jr == jj) ? x : v;
        }
        oh[16 * (2 * W * jr + mm) + 4 * qg + r] = v + zt;
      }
    }
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const float l = row_sum16(st.l[h][u]);
      const int hb = h * HS + HPL * qg + u;
      if (n == 0) {
        ml[hb * 2] = st.m[h][u];
        ml[hb * 2 + 1] = l;
      }
    }
  }
}

// Merge layout of a workgroup's wave states: a wave's output in its own lane
// order. Slot q = (h * 2W + mm) * 64 + lane (16 bytes) holds channels
// 16 (2W jr + mm) + 4 qg + 0..3 of query head h * HS + hl for lane (hl, jr, qg),
// so the waves write it, and the merge reads it, with 16-byte accesses of
// consecutive lanes (a head-major layout puts 16 lanes of a store on one LDS
// bank). The ml area stays head-major: [NH][2] floats (max, sum).

// Reorder a wave's head-major output area [NH][D] of one head set (as
// dump_state writes it) into the slot layout of W, in place. One wave: it
// issues every read before the first write, so each read sees the head-major
// data.
template <int D, int W>
__device__ __forceinline__ void head_major_to_slots(int lane, float* o) {
  constexpr int NR = Geo<D, W>::NR;
  const int n = lane & 15, qg = lane >> 4, jr = n % NR, hl = n / NR;
  f32x4 v[2 * W];
#pragma unroll
  for (int mm = 0; mm < 2 * W; ++mm)
    v[mm] = *reinterpret_cast<const f32x4*>(o + hl * D + 16 * (2 * W * jr + mm) + 4 * qg);
#pragma unroll
  for (int mm = 0; mm < 2 * W; ++mm) *reinterpret_cast<f32x4*>(o + (mm * 64 + lane) * 4) = v[mm];
}

// A wave's state in the slot layout: the values dump_state writes.
template <int D, int W, int NHS>
__device__ __forceinline__ void dump_slots(int lane, DState<D, W, NHS>& st, bool has_zero, float* o, float* ml) {
  using G = Geo<D, W>;
  constexpr int NR = G::NR, HS = G::HS, HPL = G::HPL;
  const int n = lane & 15, qg = lane >> 4, jr = n % NR;
#pragma unroll
  for (int h = 0; h < NHS; ++h) {
    float ztm[2 * W] = {};
    if (has_zero) zero_terms<D, W, NHS>(st, h, lane, ztm);
#pragma unroll
    for (int mm = 0; mm < 2 * W; ++mm) {
      const float zt = ztm[mm];
      f32x4 v = st.acc[h][mm];
#pragma unroll
      for (int jj = 1; jj < NR; ++jj) {
        const f32x4 x = st.acc[h][2 * W * jj + mm];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (jr == jj) ? x[r] : v[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = v[r] + zt;
      *reinterpret_cast<f32x4*>(o + ((h * 2 * W + mm) * 64 + lane) * 4) = v;
    }
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const float l = row_sum16(st.l[h][u]);
      const int hb = h * HS + HPL * qg + u;
      if (n == 0) {
        ml[hb * 2] = st.m[h][u];
        ml[hb * 2 + 1] = l;
      }
    }
  }
}

// The split partials of one (sequence, KV head): rows h * S + s (query head
// h of the unit, split s), D floats of unnormalised output and a (max, sum)
// pair each. They are written and read with device-coherent accesses (the
// `sc1` policy that agent-scope atomics compile to), which bypass the
// per-XCD L2s, so a workgroup on another XCD reads what was stored.
constexpr int kCoherent = 16;  // sc1
struct UnitParts {
  __amdgpu_buffer_rsrc_t o, ml;
};
template <int D>
__device__ __forceinline__ UnitParts unit_parts(const DraftParams& P, int b, int hk) {
  const size_t row0 = ((size_t)b * P.Hq + (size_t)hk * P.g) * P.S;
  const int rows = P.g * P.S;
  return UnitParts{
      __builtin_amdgcn_make_buffer_rsrc(P.part_o + row0 * D, (short)0, rows * D * 4, 0x00020000),
      __builtin_amdgcn_make_buffer_rsrc(P.part_ml + row0 * 2, (short)0, rows * 8, 0x00020000)};
}

// Merge NWV wave states in the slot layout (wave w's at o_of(w), ml_of(w))
// and store the split's partial (running max, sum and unnormalised output
// per query head of the unit). One thread per slot, every LDS load issued
// before the arithmetic. Called by all threads of the workgroup (nthreads).
template <int D, int W, int NHS, int NWV, typename OFn, typename MLFn>
__device__ __forceinline__ void merge_slots(const DraftParams& P, int b, int hk, int split, int nthreads,
                                            const OFn& o_of, const MLFn& ml_of) {
  using G = Geo<D, W>;
  constexpr int NR = G::NR, HS = G::HS;
  for (int q = threadIdx.x; q < NHS * 2 * W * 64; q += nthreads) {
    const int lane = q & 63, mm = (q >> 6) % (2 * W), h = q / (2 * W * 64);
    const int n = lane & 15, qg = lane >> 4, jr = n % NR, head = h * HS + n / NR;
    if (head >= P.g) continue;  // padding heads of the last head set
    f32x4 ow[NWV];
    float mw[NWV], lw[NWV];
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      ow[w] = *reinterpret_cast<const f32x4*>(o_of(w) + q * 4);
      mw[w] = ml_of(w)[head * 2];
      lw[w] = ml_of(w)[head * 2 + 1];
    }
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, mw[w]);
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const bool ok = mw[w] != kNegInf;
        const float a = ok ? fast_exp2(mw[w] - M) : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) O[r] = ok ? O[r] + ow[w][r] * a : O[r];
        L = ok ? L + lw[w] * a : L;
      }
    }
    const int c0 = 16 * (2 * W * jr + mm) + 4 * qg;
    const int row = head * P.S + split;  // among the unit's partial rows
    const UnitParts up = unit_parts<D>(P, b, hk);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(O[0]), __float_as_uint(O[1]), __float_as_uint(O[2]), __float_as_uint(O[3])}, up.o,
        (row * D + c0) * 4, 0, kCoherent);
    if (c0 == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(M), __float_as_uint(L)}, up.ml, row * 8, 0,
                                            kCoherent);
  }
}

// The split merge of finish_unit, every partial load of a thread in flight
// at once. Task t < Q * SG takes the 4-channel run q = t mod Q of the unit's
// outputs (Q = g D / 4: query head q / (D / 4), channels 4 (q mod D / 4) +
// 0..3) and split group sg = t / Q, splits [sg SPG, (sg + 1) SPG), with
// SG = min(ceil(S / 16), nthreads / Q) groups of SPG splits (one group, and
// several tasks per thread, when Q > nthreads), loaded BATCH (<= SPG, or 16)
// at a time: up to 16 splits in one trip to memory, without the group merge
// through LDS. A task merges its splits in split order; with one group it stores
// the run, else it leaves (max, sum, run) in LDS and thread q < Q merges the
// SG groups in group order. The order of the additions depends on S and the
// workgroup size only, never on which workgroup merges. lds: nthreads * 6
// floats, free.
struct MergeGroups {
  int Q, SG, SPG;
};
template <int D>
__device__ __forceinline__ MergeGroups merge_groups(const DraftParams& P, int nthreads) {
  const int Q = P.g * (D / 4);
  const int SG = max(1, min((P.S + 15) / 16, nthreads / Q));
  return MergeGroups{Q, SG, (P.S + SG - 1) / SG};
}
template <int D, int BATCH>
__device__ __forceinline__ void merge_unit(const DraftParams& P, int b, int hk, int nthreads, float* lds) {
  constexpr int QPH = D / 4;
  const MergeGroups mg = merge_groups<D>(P, nthreads);
  const int Q = mg.Q, SG = mg.SG, SPG = mg.SPG;
  const UnitParts up = unit_parts<D>(P, b, hk);
  float* const out = P.out + ((size_t)b * P.Hq + (size_t)hk * P.g) * D;
  auto finish = [&](int q, const f32x4& O, float L) {
    *reinterpret_cast<f32x4*>(out + 4 * q) = L > 0.f ? O / L : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  for (int t = threadIdx.x; t < Q * SG; t += nthreads) {
    const int q = t % Q, sg = t / Q, h = q / QPH, c4 = q % QPH;
    const int s0 = sg * SPG, s1 = min(P.S, s0 + SPG);
    float M = kNegInf, L = 0.f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sb = s0; sb < s1; sb += BATCH) {
      u32x4 o[BATCH];
      u32x2 ml[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int row = h * P.S + min(sb + i, s1 - 1);  // past the group: its last split again, unused
        o[i] = __builtin_amdgcn_raw_buffer_load_b128(up.o, (row * D + 4 * c4) * 4, 0, kCoherent);
        ml[i] = __builtin_amdgcn_raw_buffer_load_b64(up.ml, row * 8, 0, kCoherent);
      }
      float m[BATCH];
      float mx = M;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        m[i] = sb + i < s1 ? __uint_as_float(ml[i][0]) : kNegInf;
        mx = fmaxf(mx, m[i]);
      }
      if (mx == kNegInf) continue;  // nothing visible so far
      const float a = M == kNegInf ? 0.f : fast_exp2(M - mx);
      O *= a;
      L *= a;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const bool ok = m[i] != kNegInf;
        const float w = ok ? fast_exp2(m[i] - mx) : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) O[r] = ok ? fmaf(__uint_as_float(o[i][r]), w, O[r]) : O[r];
        L = ok ? fmaf(__uint_as_float(ml[i][1]), w, L) : L;
      }
      M = mx;
    }
    if (SG == 1) {
      finish(q, O, L);
    } else {
      float* g = lds + (size_t)t * 6;  // t < nthreads here
      *reinterpret_cast<f32x4*>(g) = O;
      g[4] = M;
      g[5] = L;
    }
  }
  if (SG == 1) return;
  __syncthreads();
  const int q = threadIdx.x;
  if (q >= Q) return;
  float M = kNegInf;
  for (int sg = 0; sg < SG; ++sg) M = fmaxf(M, lds[(sg * Q + q) * 6 + 4]);
  f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != kNegInf) {
    for (int sg = 0; sg < SG; ++sg) {
      const float* g = lds + (size_t)(sg * Q + q) * 6;
      if (g[4] == kNegInf) continue;
      const float w = fast_exp2(g[4] - M);
      const f32x4 og = *reinterpret_cast<const f32x4*>(g);
#pragma unroll
      for (int r = 0; r < 4; ++r) O[r] = fmaf(og[r], w, O[r]);
      L = fmaf(g[5], w, L);
    }
  }
  finish(q, O, L);
}

// Called by every thread after merge_slots. The workgroup's partial stores
// complete, then one thread counts the split in; the workgroup that brings
// the count to S merges the S partials of its (sequence, KV head) in a fixed
// order (so the result does not depend on the order in which workgroups
// ran), writes the output and sets the count back to zero for the next
// call. The partials are written and read with device-coherent accesses
// (they bypass the per-XCD L2s), and every thread waits for its stores to
// complete (vmcnt(0)) before the workgroup barrier that precedes the counter
// atomic, so the partials are in coherent memory before the count can reach
// S. A release on the counter atomic and an acquire fence in the merging
// workgroup would state that ordering in the memory model, but at agent
// scope on MI355X they write back and invalidate the L2: measured, the draft
// kernel went from 41.2 to 54.2 us per launch on the Llama-3-8B layer and
// from 135.2 to 146.8 us on the Qwen-32B layer.
template <int D>
__device__ __forceinline__ void finish_unit(const DraftParams& P, int b, int hk, int nthreads, int* lds_flag,
                                            float* lds) {
  const size_t unit = (size_t)b * P.Hkv + hk;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(&P.counters[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = before == (uint32_t)(P.S - 1);
  }
  __syncthreads();
  if (!*lds_flag) return;
  asm volatile("" ::: "memory");
  // a load batch no larger than a task's splits (loads past them would be
  // issued for nothing)
  const int spg = merge_groups<D>(P, nthreads).SPG;
  if (spg <= 1)
    merge_unit<D, 1>(P, b, hk, nthreads, lds);
  else if (spg <= 2)
    merge_unit<D, 2>(P, b, hk, nthreads, lds);
  else if (spg <= 4)
    merge_unit<D, 4>(P, b, hk, nthreads, lds);
  else if (spg <= 8)
    merge_unit<D, 8>(P, b, hk, nthreads, lds);
  else
    merge_unit<D, 16>(P, b, hk, nthreads, lds);
  if (threadIdx.x == 0) __hip_atomic_store(&P.counters[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the NW wave states of a row-kernel workgroup, store the split's
// partial and take part in the split merge. lds must hold NW * NH * (D + 2)
// floats; it may alias the row staging area (the leading barrier orders the
// reuse).
template <int D, int NHS, int NW>
__device__ __forceinline__ void store_partial(const DraftParams& P, int b, int hk, int split, int lane, int wave,
                                              DState<D, 1, NHS>& st, float* lds) {
  constexpr int NH = NHS * Geo<D, 1>::HS;
  float* lds_o = lds;
  float* lds_ml = lds + NW * NH * D;
  __syncthreads();
  dump_slots<D, 1, NHS>(lane, st, false, lds_o + (size_t)wave * NH * D, lds_ml + wave * NH * 2);
  __syncthreads();
  merge_slots<D, 1, NHS, NW>(
      P, b, hk, split, 64 * NW, [&](int w) { return lds_o + (size_t)w * NH * D; },
      [&](int w) { return lds_ml + w * NH * 2; });
  __shared__ int last;
  finish_unit<D>(P, b, hk, 64 * NW, &last, lds);
}

template <int D>
struct PlainRows {
  const uint16_t *kb, *vb;
  __device__ __forceinline__ const uint16_t* k(int t, int) const { return kb + (size_t)t * D; }
  __device__ __forceinline__ const uint16_t* v(int t, int) const { return vb + (size_t)t * D; }
};

// Gathered rows of one block: the kept positions of the rows a lane reads
// (value rows lane / CPR + RPI u, key rows 16 i + n; a row past the block's
// end takes the last row's position), loaded into registers one block
// ahead, so a block's rows need only their own trip to memory.
template <int D>
struct KeptRows {
  static constexpr int CPR = D / 8, RPI = 64 / CPR, NV = 32 / RPI;
  const uint16_t *kb, *vb;
  int pv[NV], pk[2];
  // positions of block rows [t0, t0 + nvalid) of the unit's kept list;
  // nvalid >= 1, and every position is clamped into the source rows
  __device__ __forceinline__ void load(const int32_t* kept, int t0, int nvalid, int cap, int lane) {
    int raw_v[NV], raw_k[2];
#pragma unroll
    for (int u = 0; u < NV; ++u) raw_v[u] = kept[t0 + min(lane / CPR + RPI * u, nvalid - 1)];
#pragma unroll
    for (int i = 0; i < 2; ++i) raw_k[i] = kept[t0 + min(16 * i + (lane & 15), nvalid - 1)];
#pragma unroll
    for (int u = 0; u < NV; ++u) pv[u] = min((int)((unsigned)raw_v[u]), cap - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) pk[i] = min((int)((unsigned)raw_k[i]), cap - 1);
  }
  __device__ __forceinline__ const uint16_t* k(int, int i) const { return kb + (size_t)pk[i] * D; }
  __device__ __forceinline__ const uint16_t* v(int, int u) const { return vb + (size_t)pv[u] * D; }
};

// Waves of a row-kernel workgroup (token drop, dense): as many as the
// kernel's registers allow on a CU, so one workgroup fills it (a CU running
// two workgroups serves the older one first), paced like the KIVI body waves.
template <int D, int NHS>
struct RowShape {
  static constexpr int PER_SIMD = D == 128 ? (NHS == 1 ? 3 : NHS <= 3 ? 2 : 1) : (NHS <= 2 ? 4 : NHS == 3 ? 3 : 2);
  static constexpr int NW = 4 * PER_SIMD;
};

// LDS of the row kernel: the row staging area (aliased by the wave merge),
// then the per-wave probability hand-over areas.
template <int D, int NHS, int NW>
constexpr size_t draft_stage_bytes() {
  constexpr int NH = NHS * Geo<D, 1>::HS;
  constexpr size_t part = (size_t)NW * NH * (D + 2) * sizeof(float);
  constexpr size_t rows = (size_t)NW * 32 * (D + 4) * sizeof(uint16_t);
  return part > rows ? part : rows;
}
template <int D, int NHS, int NW>
constexpr size_t draft_lds_bytes() {
  return draft_stage_bytes<D, NHS, NW>() + (size_t)NW * p_area_words<D, 1, NHS>() * sizeof(uint32_t);
}

// ---------------------------------------------------------------- kernels ----
// This (split, wave)'s share of the 32-token tail blocks when every split
// also streams body blocks: tail block j goes to split S - 1 - (j mod S)
// (the last split holds the fewest body blocks), wave (j / S) mod NW.
template <int D, int NHS, int NW>
__device__ __forceinline__ void tail_share(const DraftParams& P, int b, int hk, int split, int wave, int lane,
                                           DState<D, 1, NHS>& st, uint16_t* lds_rows, uint32_t* lds_p) {
  const size_t unit = (size_t)b * P.Hkv + hk;
  const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
  int j = wave * P.S + (P.S - 1 - split);
  if (j * 32 >= nt) return;
  uint32_t Aqm[NHS][D / 32][4];
  row_query<D, NHS, true>(P, b, hk, lane, Aqm);
  const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
  const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
  for (; j * 32 < nt; j += P.S * NW) {
    const PlainRows<D> rows{tk + (size_t)j * 32 * D, tv + (size_t)j * 32 * D};
    row_block<D, 1, NHS, true>(rows, min(32, nt - j * 32), lane, P.qscale, Aqm, st, lds_rows, lds_p);
  }
}

// Waves of a KIVI workgroup: NW body waves stream the quantised blocks, one
// more wave takes the fp16 tail. A workgroup holds a whole CU (its LDS ring
// or its registers leave no room for a second): a CU running two workgroups
// serves the older one first, so its younger one ends long after the older
// and the last part of the launch runs on half the waves. NW is eight where
// three waves of the kernel fit one SIMD's registers, three where only one
// does (four channel groups per MFMA row).
template <int D, int BITS, int W>
struct KiviShape {
  static constexpr int NW = (D == 128 && W == 4) ? 3 : 8;
  static_assert(NW <= 8, "progress slots");
  static constexpr int THREADS = 64 * (NW + 1);
  static constexpr int MIN_WAVES = (NW + 1 + 3) / 4;  // waves per SIMD the registers must allow
  // heads of the wave-merge layout: the body head set, which the tail's
  // one-group head sets cover exactly
  static constexpr int NHS1 = (Geo<D, W>::HS + Geo<D, 1>::HS - 1) / Geo<D, 1>::HS;
  static constexpr int NH = Geo<D, W>::HS;
  static_assert(NHS1 * Geo<D, 1>::HS == NH, "tail head sets");
};

// LDS of the KIVI kernel: NS ring stages (one per variable, so the compiler
// can tell which pending direct-to-LDS loads a read depends on; the first
// also hosts the body waves' merge layout at the end), the tail wave's merge
// layout and row staging, then the probability areas.
template <int D, int BITS, int W>
struct KiviLds {
  static constexpr int NW = KiviShape<D, BITS, W>::NW, NH = KiviShape<D, BITS, W>::NH;
  static constexpr int STAGE = NW * BlockLayout<D, BITS>::BYTES;
  // ring depth for one-group rows: six stages (four blocks in flight per
  // wave) while they fit in 150 KB; wider rows do more work per block and
  // keep three stages
  static constexpr int NS = (W == 1 && 6 * STAGE <= 150 * 1024) ? 6 : 3;
  static constexpr int MERGE = NW * NH * (D + 2) * 4;
  static constexpr int STAGE0 = STAGE > MERGE ? STAGE : MERGE;
  static constexpr int TAIL = NH * (D + 2) * 4;
  static constexpr int PAREA = p_area_words<D, W, 1>();  // per wave, words
  static_assert(p_area_words<D, 1, KiviShape<D, BITS, W>::NHS1>() == PAREA, "probability area");
};

// KIVI body + fp16 tail, one head set of HS = 16*W/NG >= g query heads. The
// body blocks of a (sequence, KV head) are cut into P.S ranges of NW * P.bpw
// blocks, one per workgroup; tail block j goes to the tail wave of workgroup
// j mod P.S.
template <int D, int BITS, int W>
__global__ __launch_bounds__((KiviShape<D, BITS, W>::THREADS), (KiviShape<D, BITS, W>::MIN_WAVES)) void draft_kivi_kernel(
    const DraftParams P) {
  using BL = BlockLayout<D, BITS>;
  using LL = KiviLds<D, BITS, W>;
  constexpr int NW = LL::NW, NH = LL::NH, NHS1 = KiviShape<D, BITS, W>::NHS1;
  __shared__ __attribute__((aligned(16))) char rs0[LL::STAGE0];
  __shared__ __attribute__((aligned(16))) char rs1[LL::STAGE];
  __shared__ __attribute__((aligned(16))) char rs2[LL::STAGE];
  __shared__ __attribute__((aligned(16))) char rs3[LL::NS > 3 ? LL::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char rs4[LL::NS > 3 ? LL::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char rs5[LL::NS > 3 ? LL::STAGE : 16];
  __shared__ __attribute__((aligned(16))) float tail_merge[LL::TAIL / 4];
  __shared__ __attribute__((aligned(16))) uint16_t tail_rows[32 * (D + 4)];
  __shared__ __attribute__((aligned(16))) uint32_t parea[(NW + 1) * LL::PAREA];
  __shared__ __attribute__((aligned(16))) int progress[8];  // blocks each body wave has started
  // the wave index is uniform across the wave; saying so keeps the per-block
  // offsets in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  uint32_t* lds_p = parea + wave * LL::PAREA;
  float* const body_o = reinterpret_cast<float*>(rs0);
  float* const body_ml = body_o + NW * NH * D;

  if (threadIdx.x < 8) progress[threadIdx.x] = 0;
  __syncthreads();

  DState<D, W, 1> st;
  st.init();
  if (wave < NW) {
    // two body waves share each SIMD: the one behind is given the issue
    // slots first, so the body waves end together
    const uint32_t prog_lds = lds_addr(progress);
    auto pace = [&](int i) { pace_waves<NW>(prog_lds, wave, i); };
    // The body length (a scalar load, on a counter the ring's loads do not
    // wait on) and the query go out first; the ring starts before either has
    // arrived.
    const int blen = ((const __attribute__((address_space(4))) int*)(P.body_len))[b];
    KiviQueryRaw<D, W> qraw;
    kivi_query_load<D, W>(P, b, hk, lane, qraw);
    KiviQuery<D, W> Q;
    // the workgroup's blocks [g0, g1) are dealt to its body waves in turn
    // (wave w takes g0 + w, g0 + w + NW, ...), so the waves of a workgroup
    // read neighbouring records; i counts this wave's blocks
    const int nbc = P.body_cap / 32;
    const int g0 = split * NW * P.bpw;
    auto gblk = [&](int i) { return g0 + wave + NW * i; };
    auto count = [&](int nb) { return max(0, (min(g0 + NW * P.bpw, nb) - g0 - wave + NW - 1) / NW); };
    // the first NS - 1 loads are issued for the range a full body would
    // give (cnt <= cnt_cap). They agree with the real range up to the wave's
    // last block; a stage past it is never computed on, and every load stays
    // inside the unit's records.
    const int cnt_cap = count(nbc);
    KiviRes res;
    res.blocks = make_rsrc(P.kivi_blocks + unit * (size_t)nbc * BL::BYTES, (size_t)nbc * BL::BYTES);
    constexpr int NS = LL::NS;
    char* const w0 = rs0 + wave * BL::BYTES;
    char* const w1 = rs1 + wave * BL::BYTES;
    char* const w2 = rs2 + wave * BL::BYTES;
    char* const w3 = rs3 + (NS > 3 ? wave * BL::BYTES : 0);
    char* const w4 = rs4 + (NS > 3 ? wave * BL::BYTES : 0);
    char* const w5 = rs5 + (NS > 3 ? wave * BL::BYTES : 0);
    if (cnt_cap > 0) {
      const int last_cap = cnt_cap - 1;
      issue_block<D, BITS>(w0, res, gblk(0), lane);
      issue_block<D, BITS>(w1, res, gblk(min(1, last_cap)), lane);
      if constexpr (NS == 6) {
        issue_block<D, BITS>(w2, res, gblk(min(2, last_cap)), lane);
        issue_block<D, BITS>(w3, res, gblk(min(3, last_cap)), lane);
        issue_block<D, BITS>(w4, res, gblk(min(4, last_cap)), lane);
      }
      const int cnt = count(min(max(blen, 0), P.body_cap) / 32);
      // NS-stage ring, loads issued NS - 1 blocks ahead; the operands of a
      // later block move from LDS to registers at the end of a step, so their
      // latency overlaps the step's last MFMAs. Past the wave's last block
      // the last one is loaded again (into a stage that is not read), which
      // keeps every wait count constant. A wave whose real range is empty
      // runs one step on its first speculative block and drops it below.
      const int b0 = 0, last = max(cnt - 1, 0);
      KiviRaw<D, BITS, W> ra, rb;
      if constexpr (NS == 6) {
        // three register sets: the operands of block i + 2 are read while
        // block i is computed, so the LDS reads have a whole step to land
        KiviRaw<D, BITS, W> rc;
        auto step3 = [&](const KiviRaw<D, BITS, W>& cur, const char* cur_stage, KiviRaw<D, BITS, W>& nxt2,
                         char* refill, int refill_blk, const char* stage2, bool paced) {
          const f32x4 cb = kivi_zero_term<D, BITS, W>(cur_stage, lane, Q);
          issue_block<D, BITS>(refill, res, gblk(min(refill_blk, last)), lane);
          if (paced) pace(refill_blk - 5);
          kivi_compute<D, BITS, W>(cur, cb, lane, Q, st, lds_p);
          wait_vm<3 * BL::NI>();  // block i + 2 has landed
          kivi_read<D, BITS, W>(nxt2, stage2, lane);
        };
        kivi_query_finish<D, W>(P, lane, qraw, Q);
        wait_vm<3 * BL::NI>();
        kivi_read<D, BITS, W>(ra, w0, lane);
        kivi_read<D, BITS, W>(rb, w1, lane);
        for (int blk = b0;; blk += 6) {
          // block i sits in stage i mod 6
          step3(ra, w0, rc, w5, blk + 5, w2, true);
          if (blk + 1 > last) break;
          step3(rb, w1, ra, w0, blk + 6, w3, false);
          if (blk + 2 > last) break;
          step3(rc, w2, rb, w1, blk + 7, w4, true);
          if (blk + 3 > last) break;
          step3(ra, w3, rc, w2, blk + 8, w5, false);
          if (blk + 4 > last) break;
          step3(rb, w4, ra, w3, blk + 9, w0, true);
          if (blk + 5 > last) break;
          step3(rc, w5, rb, w4, blk + 10, w1, false);
          if (blk + 6 > last) break;
        }
      } else {
        // paced once per six blocks (measured against every second and
        // third block: Qwen-32B layer 132.8 / 132.4 -> 131.1 us; the
        // six-stage path above keeps every second block: Llama-3-8B layer
        // 40.9 against 41.3 us once per six)
        auto step = [&](const KiviRaw<D, BITS, W>& cur, const char* cur_stage, KiviRaw<D, BITS, W>& nxt,
                        char* refill, int refill_blk, const char* next_stage, bool paced) {
          // the zero-point term reads the block's stage before the refill
          // is issued (only the next block's load is then in flight)
          const f32x4 cb = kivi_zero_term<D, BITS, W>(cur_stage, lane, Q);
          issue_block<D, BITS>(refill, res, gblk(min(refill_blk, last)), lane);
          if (paced) pace(refill_blk - 2);
          kivi_compute<D, BITS, W>(cur, cb, lane, Q, st, lds_p);
          wait_vm<(NS - 2) * BL::NI>();  // the next block has landed
          kivi_read<D, BITS, W>(nxt, next_stage, lane);
        };
        kivi_query_finish<D, W>(P, lane, qraw, Q);
        wait_vm<BL::NI>();
        kivi_read<D, BITS, W>(ra, w0, lane);
        for (int blk = b0;; blk += 6) {
          // block i sits in stage i mod 3
          step(ra, w0, rb, w2, blk + 2, w1, true);
          if (blk + 1 > last) break;
          step(rb, w1, ra, w0, blk + 3, w2, false);
          if (blk + 2 > last) break;
          step(ra, w2, rb, w1, blk + 4, w0, false);
          if (blk + 3 > last) break;
          step(rb, w0, ra, w2, blk + 5, w1, false);
          if (blk + 4 > last) break;
          step(ra, w1, rb, w0, blk + 6, w2, false);
          if (blk + 5 > last) break;
          step(rb, w2, ra, w1, blk + 7, w0, false);
          if (blk + 6 > last) break;
        }
      }
      // every ring load has landed before the ring's memory is reused
      wait_vm<0>();
      // a wave whose real range is empty (a body shorter than its
      // capacity) computed its first speculative block: drop it
      if (cnt == 0) st.init();
    }
  } else {
    // the tail wave: fp16 rows with the values staged in LDS (so a block
    // takes one trip to memory), one-group rows (a separate state whose head
    // sets cover the body head set), written to its own merge area at once
    DState<D, 1, NHS1> st1;
    st1.init();
    uint32_t Aqm[NHS1][D / 32][4];
    row_query<D, NHS1, false>(P, b, hk, lane, Aqm);
    const int nt = min(max(P.tail_len[b], 0), P.tail_cap);
    const uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
    const uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
    for (int blk = split; blk * 32 < nt; blk += P.S) {
      const PlainRows<D> rows{tk + (size_t)blk * 32 * D, tv + (size_t)blk * 32 * D};
      row_block<D, 1, NHS1, false>(rows, min(32, nt - blk * 32), lane, P.qscale, Aqm, st1, tail_rows, lds_p);
    }
    dump_state<D, 1, NHS1>(lane, st1, false, tail_merge, tail_merge + NH * D);
    head_major_to_slots<D, W>(lane, tail_merge);
  }
  // the ring (and with it the body waves' merge area) is free once every body
  // wave has left its loop
  __syncthreads();
  if (wave < NW) dump_slots<D, W, 1>(lane, st, true, body_o + (size_t)wave * NH * D, body_ml + wave * NH * 2);
  __syncthreads();
  merge_slots<D, W, 1, NW + 1>(
      P, b, hk, split, LL::NW * 64 + 64,
      [&](int w) { return w < NW ? body_o + (size_t)w * NH * D : tail_merge; },
      [&](int w) { return w < NW ? body_ml + w * NH * 2 : tail_merge + NH * D; });
  static_assert(LL::STAGE0 >= (LL::NW * 64 + 64) * 6 * 4, "split merge area");
  __shared__ int last;
  finish_unit<D>(P, b, hk, LL::NW * 64 + 64, &last, body_o);
}

// Token-drop (GATHER) and dense draft caches: bf16 rows everywhere. The
// split's blocks [g0, g1) are dealt to its NW waves in turn (wave w takes
// g0 + w, g0 + w + NW, ...), then every wave takes its share of the tail.
template <int D, int NHS, bool GATHER>
__global__ __launch_bounds__((64 * RowShape<D, NHS>::NW), (RowShape<D, NHS>::PER_SIMD)) void draft_rows_kernel(
    const DraftParams P) {
  constexpr int NW = RowShape<D, NHS>::NW;
  __shared__ __attribute__((aligned(16))) char smem[draft_lds_bytes<D, NHS, NW>()];
  __shared__ __attribute__((aligned(16))) int progress[16];  // blocks each wave has started
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  uint32_t* lds_p =
      reinterpret_cast<uint32_t*>(smem + draft_stage_bytes<D, NHS, NW>()) + wave * p_area_words<D, 1, NHS>();
  if (threadIdx.x < 16) progress[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prog_lds = lds_addr(progress);

  DState<D, 1, NHS> st;
  st.init();
  uint32_t Aqm[NHS][D / 32][4];
  row_query<D, NHS, true>(P, b, hk, lane, Aqm);
  uint16_t* my_lds = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 4);
  {
    const int nb = min(max(P.body_len[b], 0), P.body_cap);
    const int nblk = (nb + 31) / 32;
    const int g0 = split * NW * P.bpw;
    const int g1 = min(g0 + NW * P.bpw, nblk);
    const uint16_t* sk = P.src_k + unit * (size_t)P.src_t_cap * D;
    const uint16_t* sv = P.src_v + unit * (size_t)P.src_t_cap * D;
    int i = 0;
    if constexpr (GATHER) {
      const int32_t* kept = P.kept_idx + unit * (size_t)P.body_cap;
      KeptRows<D> cur{sk, sv}, nxt{sk, sv};
      if (g0 + wave < g1) cur.load(kept, (g0 + wave) * 32, min(32, nb - (g0 + wave) * 32), P.src_t_cap, lane);
      for (int blk = g0 + wave; blk < g1; blk += NW, ++i) {
        // the next block's positions (this block's again after the last)
        const int nb2 = min(blk + NW, g1 - 1);
        nxt.load(kept, nb2 * 32, min(32, nb - nb2 * 32), P.src_t_cap, lane);
        pace_waves<NW>(prog_lds, wave, i);
        row_block<D, 1, NHS, true>(cur, min(32, nb - blk * 32), lane, P.qscale, Aqm, st, my_lds, lds_p);
        cur = nxt;
      }
    } else {
      for (int blk = g0 + wave; blk < g1; blk += NW, ++i) {
        // paced every fourth block (the dense full-KV pass, measured against
        // every block: Mistral-24B layer 361.7 -> 346.5 us, Qwen-32B layer
        // 699.4 -> 690.0 us; the gathered blocks above are faster paced
        // every block: 94.9 against 99.3 us)
        if ((i & 3) == 0) pace_waves<NW>(prog_lds, wave, i);
        const PlainRows<D> rows{sk + (size_t)blk * 32 * D, sv + (size_t)blk * 32 * D};
        row_block<D, 1, NHS, true>(rows, min(32, nb - blk * 32), lane, P.qscale, Aqm, st, my_lds, lds_p);
      }
    }
  }
  tail_share<D, NHS, NW>(P, b, hk, split, wave, lane, st, my_lds, lds_p);
  static_assert(draft_stage_bytes<D, NHS, NW>() >= 64 * NW * 6 * sizeof(float), "split merge area");
  store_partial<D, NHS, NW>(P, b, hk, split, lane, wave, st, reinterpret_cast<float*>(smem));
}

// Head sets of the row kernel (W = 1).
template <int D>
int pick_nhs(int g) {
  constexpr int HS = Geo<D, 1>::HS;
  return (g + HS - 1) / HS;
}
// Row width of the KIVI kernel: the narrowest W whose head set holds g heads.
template <int D>
int pick_w(int g) {
  constexpr int NG = D / 32;
  int w = 1;
  while (w < NG && 16 * w / NG < g) w *= 2;
  return w;
}

using DraftKernel = void (*)(DraftParams);

// A kernel with its workgroup shape: waves that stream body blocks (nw) and
// threads per workgroup.
struct DraftKernelPick {
  DraftKernel fn;
  int nw, threads;
};

template <int D, int BITS, int W>
DraftKernelPick kivi_pick() {
  return DraftKernelPick{draft_kivi_kernel<D, BITS, W>, KiviShape<D, BITS, W>::NW, KiviShape<D, BITS, W>::THREADS};
}
template <int D, int BITS>
DraftKernelPick kivi_kernel_for(int w) {
  if constexpr (D == 128) {
    switch (w) {
      case 1: return kivi_pick<D, BITS, 1>();
      case 2: return kivi_pick<D, BITS, 2>();
      default: return kivi_pick<D, BITS, 4>();
    }
  } else {
    return w == 1 ? kivi_pick<D, BITS, 1>() : kivi_pick<D, BITS, 2>();
  }
}
template <int D, bool GATHER>
DraftKernelPick rows_kernel_for(int nhs) {
  DraftKernel k;
  switch (nhs) {
    case 1: k = draft_rows_kernel<D, 1, GATHER>; break;
    case 2: k = draft_rows_kernel<D, 2, GATHER>; break;
    case 3: k = draft_rows_kernel<D, 3, GATHER>; break;
    default: k = draft_rows_kernel<D, 4, GATHER>; break;
  }
  constexpr int NW[5] = {0, RowShape<D, 1>::NW, RowShape<D, 2>::NW, RowShape<D, 3>::NW, RowShape<D, 4>::NW};
  const int nw = NW[nhs < 1 ? 1 : nhs > 4 ? 4 : nhs];
  return DraftKernelPick{k, nw, 64 * nw};
}

DraftKernelPick pick_kernel(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  const int D = sh.head_dim, g = sh.n_q_heads / sh.n_kv_heads;
  if (kv.kind == VC_DRAFT_KIVI) {
    const int w = D == 128 ? pick_w<128>(g) : pick_w<64>(g);
    if (D == 128) return kv.bits == 2 ? kivi_kernel_for<128, 2>(w) : kivi_kernel_for<128, 4>(w);
    return kv.bits == 2 ? kivi_kernel_for<64, 2>(w) : kivi_kernel_for<64, 4>(w);
  }
  const int nhs = D == 128 ? pick_nhs<128>(g) : pick_nhs<64>(g);
  if (kv.kind == VC_DRAFT_TOKDROP) return D == 128 ? rows_kernel_for<128, true>(nhs) : rows_kernel_for<64, true>(nhs);
  return D == 128 ? rows_kernel_for<128, false>(nhs) : rows_kernel_for<64, false>(nhs);
}

// Workgroups of kernel k that the current device holds at once (CUs times
// workgroups per CU), cached per (device, kernel). Without a device (a
// workspace query on a host with no GPU) four per CU of a 256-CU part are
// assumed, which is at least what any draft kernel holds, so such a
// workspace is large enough.
long long resident_wgs(const DraftKernelPick& k) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, long long> cache;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256 * 4;
  }
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, reinterpret_cast<const void*>(k.fn));
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k.fn), k.threads, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256 * 4;
  }
  const long long n = (long long)(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  cache[key] = n;
  return n;
}

}  // namespace

// Split plan shared by the workspace query and the launch: as many splits as
// let every workgroup be resident at once, so the kernel runs in one round.
struct DraftPlan {
  int bpw;     // body blocks per body wave
  int splits;  // workgroups per (sequence, KV head)
};

// The splits of every (sequence, KV head) fill the resident workgroups once;
// each split takes a range of nw * bpw body blocks and a share of the tail
// (the KIVI kernel gives its share to a wave of its own, the row kernels
// stage it like the body).
DraftPlan draft_plan(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  const long long blocks = (kv.body_cap + 31) / 32;
  const long long units = (long long)sh.batch * sh.n_kv_heads;
  const DraftKernelPick k = pick_kernel(sh, kv);
  long long splits = resident_wgs(k) / units;
  if (splits < 1) splits = 1;
  long long bpw = (blocks + splits * k.nw - 1) / (splits * k.nw);
  if (bpw < 1) bpw = 1;
  splits = (blocks + k.nw * bpw - 1) / (k.nw * bpw);
  if (splits < 1) splits = 1;
  return DraftPlan{(int)bpw, (int)splits};
}

// Workspace: the split counters (one 32-bit word per (sequence, KV head),
// zero between calls), then the split partials (unnormalised outputs, then
// max and sum).
size_t draft_counter_bytes(const vc_attn_shape& sh) {
  return align_up((size_t)sh.batch * sh.n_kv_heads * sizeof(uint32_t), 256);
}
size_t draft_ws_bytes(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  const DraftPlan p = draft_plan(sh, kv);
  const size_t rows = (size_t)sh.batch * sh.n_q_heads * p.splits;
  return draft_counter_bytes(sh) + align_up(rows * sh.head_dim * sizeof(float), 256) +
         align_up(rows * 2 * sizeof(float), 256);
}

// Bytes of the split partials alone (the workspace after its counters).
size_t draft_partial_bytes(const vc_attn_shape& sh, const vc_draft_kv& kv) {
  return draft_ws_bytes(sh, kv) - draft_counter_bytes(sh);
}

// counters: one zeroed word per (sequence, KV head); partials: the split
// partials (draft_partial_bytes, 256-byte aligned).
static vc_status draft_launch_parts(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out,
                                    uint32_t* counters, char* partials, hipStream_t stream) {
  const DraftPlan plan = draft_plan(sh, kv);
  DraftParams P{};
  P.q = static_cast<const uint16_t*>(q);
  const size_t rows = (size_t)sh.batch * sh.n_q_heads * plan.splits;
  char* w = partials;
  P.counters = counters;
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
  P.kivi_blocks = static_cast<const char*>(kv.kivi_blocks);
  P.kept_idx = kv.kept_idx;
  P.src_k = static_cast<const uint16_t*>(kv.src_k);
  P.src_v = static_cast<const uint16_t*>(kv.src_v);
  P.tail_k = static_cast<const uint16_t*>(kv.tail_k);
  P.tail_v = static_cast<const uint16_t*>(kv.tail_v);

  // one kernel: the split merge happens in its last workgroup per unit, so
  // both timing scopes cover the same dispatch
  const dim3 grid(plan.splits, sh.n_kv_heads, sh.batch);
  const Timing tm = take_timing();
  const DraftKernelPick k = pick_kernel(sh, kv);
  launch_ev(k.fn, grid, dim3(k.threads), 0, stream, tm.start, tm.stop, P);
  return check_launch("draft attention");
}

vc_status draft_launch(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out, void* ws,
                       hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  return draft_launch_parts(sh, q, kv, out, reinterpret_cast<uint32_t*>(w), w + draft_counter_bytes(sh), stream);
}

// ------------------------------------------------ allocation-free variant ----
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid allocation): the draft workspace lives in this
// file-scope device array instead of a caller buffer. Each GPU the library
// runs on holds its own copy until the process ends. In host code the
// array's name is only a stand-in; its device address comes from
// hipGetSymbolAddress, taken once per device and used wherever host code
// needs the array (kernel arguments, the clearing kernel).
//
// Layout: a fixed counter region (one word for every possible (sequence, KV
// head), 255 x 255) cleared once when the device is first used and left zero
// by every completed call, then the split partials of the call. The partials
// never overlap a counter, so calls of any shape can follow each other.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
constexpr size_t kNoAllocCounterBytes = (size_t(255) * 255 * sizeof(uint32_t) + 255) / 256 * 256;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Largest partials a call may need.
size_t draft_noalloc_max_partial_bytes() { return kNoAllocScratchBytes - kNoAllocCounterBytes; }

// The draft call on this device's scratch array. On the first call for a
// device its address is looked up and the counter region is cleared by a
// kernel on `stream`, ahead of any draft kernel there.
vc_status draft_launch_noalloc(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out,
                               hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(VC_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  char* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr)
        return fail(VC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                         kNoAllocCounterBytes / sizeof(uint32_t));
      const vc_status st = check_launch("draft scratch clear");
      if (st != VC_OK) return st;
      g_scratch_ptr[dev] = ptr;
    }
    base = static_cast<char*>(g_scratch_ptr[dev]);
  }
  return draft_launch_parts(sh, q, kv, out, reinterpret_cast<uint32_t*>(base), base + kNoAllocCounterBytes, stream);
}

}  // namespace vc
