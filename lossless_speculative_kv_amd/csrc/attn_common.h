// Online-softmax state shared by the draft and verification kernels.
#pragma once
#include "vc_internal.h"

namespace vc {

constexpr float kRescaleThreshold = 8.0f;  // log2 units

// State for NC MFMA column sets of one lane. Scores arrive in the log2
// domain, already scaled by log2(e)/sqrt(D).
template <int NC, int MT>
struct SoftState {
  float m[NC];   // running max, identical on all lanes of a column
  float l[NC];   // this lane's share of sum p
  float zt[NC];  // this lane's share of sum p * value zero point (KIVI)
  f32x4 acc[NC][MT];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < NC; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
      zt[h] = 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Move the running max for a 32-token block of scores s[c][tile][r] and turn
// the scores into p = 2^(s - m) in place. The max only moves when the block
// max exceeds it by more than kRescaleThreshold (so p <= 2^8), which makes
// the rescale of the accumulators rare; the result is the same softmax.
template <int NC, int MT>
__device__ __forceinline__ void softmax_block(SoftState<NC, MT>& st, float (&s)[NC][2][4]) {
  float bm[NC];
  bool need = false;
#pragma unroll
  for (int h = 0; h < NC; ++h) {
    const float x = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                          fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
    bm[h] = max_q(x);
    need = need || (bm[h] > st.m[h] + kRescaleThreshold);
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int h = 0; h < NC; ++h) {
      const bool up = bm[h] > st.m[h] + kRescaleThreshold;
      const float alpha = up ? fast_exp2(st.m[h] - bm[h]) : 1.f;
      st.m[h] = up ? bm[h] : st.m[h];
      st.l[h] *= alpha;
      st.zt[h] *= alpha;
#pragma unroll
      for (int t = 0; t < MT; ++t) st.acc[h][t] *= alpha;
    }
  }
#pragma unroll
  for (int h = 0; h < NC; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[h][i][r] = fast_exp2(s[h][i][r] - st.m[h]);
        st.l[h] += s[h][i][r];
      }
}

// Token of PV contraction slot s (0..7) for lane group qg: the S^T tiles give
// lane group qg tokens 4*qg + r of tile 0 and 16 + 4*qg + r of tile 1.
__device__ __forceinline__ constexpr int slot_token(int qg, int s) { return 16 * (s >> 2) + 4 * qg + (s & 3); }

}  // namespace vc
