// Verification attention over the full bf16 cache (VeriCache summary, "Core
// algorithm": one forward pass with KV_full checks all drafted tokens in
// parallel; "P1": verification loads the full cache and is also
// compute-bound, since every cached token meets (k+1)*g query rows).
//
// Work decomposition: one workgroup per (context split, KV head, sequence).
// All R = n_rows * g query rows of the KV head (row = j * g + head, j the
// draft position) live in the workgroup, RT row tiles of 16 per wave, so
// each K/V tile is read from HBM once and staged in LDS (double-buffered,
// 32 tokens per stage) for every row tile.
//   QK: S^T[token][row] on v_mfma_f32_16x16x32_bf16, A = 16 key rows (from
//       LDS), B = 16 query rows (registers, exact bf16).
//   PV: O^T[channel][row] += V^T[channel][token] * P^T[token][row]; V^T is
//       read from LDS as 16-bit values (8 tokens per lane per channel).
// The draft block (x_0..x_k's own keys/values) is the last split of the END
// call, with the causal mask (row j sees block rows 0..j). Per-split
// partials (max, sum, unnormalised output) are folded in split order into a
// running state kept in the workspace, which allows the context to arrive in
// staged chunks over several calls.
#include "attn_common.h"

namespace vc {

namespace {

struct VerifyParams {
  const uint16_t* q;      // bf16 [NR][B][Hq][D]
  const uint16_t* k_new;  // bf16 [NR][B][Hkv][D]
  const uint16_t* v_new;
  const uint16_t* ck;  // chunk bf16 [u][t_cap][D]
  const uint16_t* cv;
  int t_cap, tok_begin, tok_count;
  const int32_t* ctx_len;
  float* part_o;  // [u][S][R][D]
  float* part_ml; // [u][S][R][2]
  float* run_o;   // [u][R][D]
  float* run_ml;  // [u][R][2]
  float* out;     // fp32 [NR][B][Hq][D]
  int B, Hq, Hkv, g, NR, R, S, S_ctx, tps, flags;
  float qscale;
};

constexpr int kTT = 32;  // tokens per LDS stage

template <int D>
struct VerifyLds {
  static constexpr int KSTR = D + 8;  // halfs; 16-byte aligned rows
  static constexpr int VSTR = D + 4;  // halfs; conflict-free 16-bit transposed reads
  static constexpr int KBUF = kTT * KSTR, VBUF = kTT * VSTR;
  static constexpr int BYTES = 2 * (KBUF + VBUF) * 2;
};

// Global -> register prefetch of one 32-token K/V tile. Each thread moves
// 16-byte chunks; rows of invalid tokens are zero.
template <int D, int MAXC>
struct TilePrefetch {
  u32x4 k[MAXC], v[MAXC];
};

template <int D, int MAXC, typename RowFn>
__device__ __forceinline__ void prefetch_tile(TilePrefetch<D, MAXC>& pf, const RowFn& rows, int nvalid, int tid,
                                              int nthreads) {
  constexpr int CPR = D / 8, CH = kTT * CPR;
#pragma unroll
  for (int u = 0; u < MAXC; ++u) {
    const int c = tid + u * nthreads;
    pf.k[u] = u32x4{0u, 0u, 0u, 0u};
    pf.v[u] = u32x4{0u, 0u, 0u, 0u};
    if (c < CH) {
      const int t = c / CPR, x = c % CPR;
      if (t < nvalid) {
        pf.k[u] = *reinterpret_cast<const u32x4*>(rows.k(t) + 8 * x);
        pf.v[u] = *reinterpret_cast<const u32x4*>(rows.v(t) + 8 * x);
      }
    }
  }
}

template <int D, int MAXC>
__device__ __forceinline__ void store_tile(const TilePrefetch<D, MAXC>& pf, uint16_t* kb, uint16_t* vb, int tid,
                                           int nthreads) {
  constexpr int CPR = D / 8, CH = kTT * CPR;
  using L = VerifyLds<D>;
#pragma unroll
  for (int u = 0; u < MAXC; ++u) {
    const int c = tid + u * nthreads;
    if (c < CH) {
      const int t = c / CPR, x = c % CPR;
      *reinterpret_cast<u32x4*>(kb + t * L::KSTR + 8 * x) = pf.k[u];
      uint32_t* d = reinterpret_cast<uint32_t*>(vb + t * L::VSTR + 8 * x);
      *reinterpret_cast<u32x2*>(d) = u32x2{pf.v[u][0], pf.v[u][1]};
      *reinterpret_cast<u32x2*>(d + 2) = u32x2{pf.v[u][2], pf.v[u][3]};
    }
  }
}

template <int D>
struct CtxRows {
  const uint16_t *kb, *vb;
  __device__ __forceinline__ const uint16_t* k(int t) const { return kb + (size_t)t * D; }
  __device__ __forceinline__ const uint16_t* v(int t) const { return vb + (size_t)t * D; }
};
// Block token i of sequence b: row (i, b, hk) of k_new / v_new.
template <int D>
struct BlockRows {
  const uint16_t *kb, *vb;
  int stride;  // halfs between consecutive block tokens (B * Hkv * D)
  __device__ __forceinline__ const uint16_t* k(int t) const { return kb + (size_t)t * stride; }
  __device__ __forceinline__ const uint16_t* v(int t) const { return vb + (size_t)t * stride; }
};

// One 32-token stage for this wave's RT row tiles. tok_valid(t) masks tokens
// for all rows; blk_row_min(t) >= 0 marks a block token that only rows with
// draft position j >= blk_row_min(t) may see.
template <int D, int RT, bool CAUSAL>
__device__ __forceinline__ void verify_stage(const uint16_t* kb, const uint16_t* vb, int nvalid, int lane,
                                             const uint32_t (&Bq)[RT][D / 32][4], const int (&rowj)[RT],
                                             float qscale, SoftState<RT, D / 16>& st) {
  constexpr int NG = D / 32, MT = D / 16;
  using L = VerifyLds<D>;
  const int n = lane & 15, qg = lane >> 4;
  float s[RT][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint16_t* kr = kb + (16 * i + n) * L::KSTR + qg * (D / 4);
    u32x4 A[NG];
#pragma unroll
    for (int kk = 0; kk < NG; ++kk) A[kk] = *reinterpret_cast<const u32x4*>(kr + 8 * kk);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk)
        c = mfma_bf16(A[kk], u32x4{Bq[rt][kk][0], Bq[rt][kk][1], Bq[rt][kk][2], Bq[rt][kk][3]}, c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * i + 4 * qg + r;
        bool ok = t < nvalid;
        if constexpr (CAUSAL) ok = ok && (t <= rowj[rt]);
        s[rt][i][r] = ok ? c[r] * qscale : kNegInf;
      }
    }
  }
  softmax_block<RT, MT>(st, s);
  uint32_t Bp[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r >> 1, rr = 2 * (r & 1);
      Bp[rt][r] = pack_bf16(s[rt][i][rr], s[rt][i][rr + 1]);
    }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t lo = vb[slot_token(qg, 2 * r) * L::VSTR + 16 * m + n];
      const uint32_t hi = vb[slot_token(qg, 2 * r + 1) * L::VSTR + 16 * m + n];
      A[r] = lo | (hi << 16);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      st.acc[rt][m] =
          mfma_bf16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Bp[rt][0], Bp[rt][1], Bp[rt][2], Bp[rt][3]}, st.acc[rt][m]);
  }
}

// Stream a run of 32-token tiles through the double-buffered LDS stages.
template <int D, int RT, int MAXC, bool CAUSAL, typename RowsAt>
__device__ __forceinline__ void verify_run(RowsAt rows_at, int ntiles, int nvalid_total, char* smem, int lane,
                                           int tid, int nthreads, const uint32_t (&Bq)[RT][D / 32][4],
                                           const int (&rowj)[RT], float qscale, SoftState<RT, D / 16>& st) {
  using L = VerifyLds<D>;
  uint16_t* base = reinterpret_cast<uint16_t*>(smem);
  TilePrefetch<D, MAXC> pf;
  if (ntiles > 0) prefetch_tile<D, MAXC>(pf, rows_at(0), min(kTT, nvalid_total), tid, nthreads);
  for (int t = 0; t < ntiles; ++t) {
    uint16_t* kb = base + (t & 1) * (L::KBUF + L::VBUF);
    uint16_t* vb = kb + L::KBUF;
    store_tile<D, MAXC>(pf, kb, vb, tid, nthreads);
    __syncthreads();
    if (t + 1 < ntiles) prefetch_tile<D, MAXC>(pf, rows_at(t + 1), min(kTT, nvalid_total - (t + 1) * kTT), tid, nthreads);
    verify_stage<D, RT, CAUSAL>(kb, vb, min(kTT, nvalid_total - t * kTT), lane, Bq, rowj, qscale, st);
  }
}

// MAXC: 16-byte chunks per thread per tensor for one stage, ceil(32*D/8 / threads).
template <int D, int RT, int MAXC>
__global__ __launch_bounds__(512) void verify_kernel(const VerifyParams P) {
  constexpr int NG = D / 32, MT = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[VerifyLds<D>::BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x, nthreads = blockDim.x;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  const int n = lane & 15, qg = lane >> 4;

  // query operands of this wave's row tiles (unscaled bf16, exact)
  uint32_t Bq[RT][NG][4];
  int rowj[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * (wave * RT + rt) + n;
    const bool ok = row < P.R;
    const int jj = ok ? row / P.g : 0, hl = ok ? row % P.g : 0;
    rowj[rt] = ok ? jj : -1;
    const uint16_t* qp = P.q + (((size_t)jj * P.B + b) * P.Hq + (size_t)hk * P.g + hl) * D + qg * (D / 4);
#pragma unroll
    for (int kk = 0; kk < NG; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(qp + 8 * kk);
      Bq[rt][kk][0] = v[0];
      Bq[rt][kk][1] = v[1];
      Bq[rt][kk][2] = v[2];
      Bq[rt][kk][3] = v[3];
    }
  }

  SoftState<RT, MT> st;
  st.init();
  if (split < P.S_ctx) {
    // context rows [r0, r1) of the chunk, positions tok_begin + r, visible below ctx_len
    const int ctx = P.ctx_len[b];
    const int r0 = split * P.tps;
    int r1 = min(r0 + P.tps, P.tok_count);
    r1 = min(r1, ctx - P.tok_begin);
    const int nval = max(0, r1 - r0);
    const int ntiles = (nval + kTT - 1) / kTT;
    const uint16_t* kb = P.ck + (unit * P.t_cap + r0) * D;
    const uint16_t* vb = P.cv + (unit * P.t_cap + r0) * D;
    verify_run<D, RT, MAXC, false>(
        [&](int t) { return CtxRows<D>{kb + (size_t)t * kTT * D, vb + (size_t)t * kTT * D}; }, ntiles, nval, smem,
        lane, tid, nthreads, Bq, rowj, P.qscale, st);
  } else {
    // the draft block: tokens x_0..x_{NR-1}, causal
    const int stride = P.B * P.Hkv * D;
    const uint16_t* kb = P.k_new + ((size_t)b * P.Hkv + hk) * D;
    const uint16_t* vb = P.v_new + ((size_t)b * P.Hkv + hk) * D;
    const int ntiles = (P.NR + kTT - 1) / kTT;
    // causal masks need the block-token index, which is tile * 32 + t; shift rowj per tile
    int rj[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rj[rt] = rowj[rt];
    using L = VerifyLds<D>;
    uint16_t* base = reinterpret_cast<uint16_t*>(smem);
    TilePrefetch<D, MAXC> pf;
    for (int t = 0; t < ntiles; ++t) {
      const BlockRows<D> rows{kb + (size_t)t * kTT * stride, vb + (size_t)t * kTT * stride, stride};
      const int nv = min(kTT, P.NR - t * kTT);
      prefetch_tile<D, MAXC>(pf, rows, nv, tid, nthreads);
      uint16_t* kbuf = base + (t & 1) * (L::KBUF + L::VBUF);
      __syncthreads();
      store_tile<D, MAXC>(pf, kbuf, kbuf + L::KBUF, tid, nthreads);
      __syncthreads();
      verify_stage<D, RT, true>(kbuf, kbuf + L::KBUF, nv, lane, Bq, rj, P.qscale, st);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) rj[rt] -= kTT;
    }
  }

  // partial for this split: rows of this wave
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * (wave * RT + rt) + n;
    const float l = sum_q(st.l[rt]);
    if (row < P.R) {
      const size_t pr = (unit * P.S + split) * P.R + row;
      float* o = P.part_o + pr * D;
#pragma unroll
      for (int m = 0; m < MT; ++m) *reinterpret_cast<f32x4*>(o + 16 * m + 4 * qg) = st.acc[rt][m];
      if (qg == 0) {
        P.part_ml[pr * 2] = st.m[rt];
        P.part_ml[pr * 2 + 1] = l;
      }
    }
  }
}

// Fold this call's splits (in order) into the running state; on END write out.
template <int D>
__global__ __launch_bounds__(D) void verify_merge_kernel(const VerifyParams P) {
  const int c = threadIdx.x, row = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  const size_t rr = unit * P.R + row;
  float M = kNegInf, L = 0.f, O = 0.f;
  if (!(P.flags & VC_VERIFY_BEGIN)) {
    M = P.run_ml[rr * 2];
    L = P.run_ml[rr * 2 + 1];
    O = P.run_o[rr * D + c];
  }
  for (int s = 0; s < P.S; ++s) {
    const size_t pr = (unit * P.S + s) * P.R + row;
    const float ms = P.part_ml[pr * 2];
    if (ms == kNegInf) continue;
    const float ls = P.part_ml[pr * 2 + 1], os = P.part_o[pr * D + c];
    if (ms > M) {
      const float a = fast_exp2(M - ms);  // 0 when M is -inf
      O = O * a + os;
      L = L * a + ls;
      M = ms;
    } else {
      const float a = fast_exp2(ms - M);
      O += os * a;
      L += ls * a;
    }
  }
  if (P.flags & VC_VERIFY_END) {
    const int j = row / P.g, hl = row % P.g;
    P.out[(((size_t)j * P.B + b) * P.Hq + (size_t)hk * P.g + hl) * D + c] = (L > 0.f) ? O / L : 0.f;
  } else {
    P.run_o[rr * D + c] = O;
    if (c == 0) {
      P.run_ml[rr * 2] = M;
      P.run_ml[rr * 2 + 1] = L;
    }
  }
}

template <int D, int RT>
void launch_verify_rt(const VerifyParams& P, int nwaves, dim3 grid, hipStream_t s) {
  const dim3 block(64 * nwaves);
  const int chunks = kTT * D / 8;
  const int maxc = (chunks + 64 * nwaves - 1) / (64 * nwaves);
  if (maxc > 4) hipLaunchKernelGGL((verify_kernel<D, RT, (kTT * D / 8 + 63) / 64>), grid, block, 0, s, P);
  else if (maxc > 2) hipLaunchKernelGGL((verify_kernel<D, RT, 4>), grid, block, 0, s, P);
  else if (maxc > 1) hipLaunchKernelGGL((verify_kernel<D, RT, 2>), grid, block, 0, s, P);
  else hipLaunchKernelGGL((verify_kernel<D, RT, 1>), grid, block, 0, s, P);
}

template <int D>
void launch_verify(const VerifyParams& P, int rt, int nwaves, dim3 grid, hipStream_t s) {
  switch (rt) {
    case 1: launch_verify_rt<D, 1>(P, nwaves, grid, s); break;
    case 2: launch_verify_rt<D, 2>(P, nwaves, grid, s); break;
    case 3: launch_verify_rt<D, 3>(P, nwaves, grid, s); break;
    default: launch_verify_rt<D, 4>(P, nwaves, grid, s); break;
  }
}

}  // namespace

struct VerifyPlan {
  int rt, nwaves, tps, s_ctx;
};

// Row tiling: up to 8 waves with RT = ceil(tiles / 8) row tiles each (<= 4).
// Context split of a call: about 512 workgroups, whole 256-token runs.
VerifyPlan verify_plan(const vc_attn_shape& sh, int n_rows, int chunk_tokens) {
  const int R = n_rows * (sh.n_q_heads / sh.n_kv_heads);
  const int tiles = (R + 15) / 16;
  int rt = (tiles + 7) / 8;
  if (rt < 1) rt = 1;
  const int nwaves = (tiles + rt - 1) / rt;
  const long long units = (long long)sh.batch * sh.n_kv_heads;
  long long tps = ((long long)chunk_tokens * units + 511) / 512;
  tps = ((tps + 255) / 256) * 256;
  if (tps < 256) tps = 256;
  int s_ctx = (int)((chunk_tokens + tps - 1) / tps);
  if (s_ctx < 1) s_ctx = 1;
  return VerifyPlan{rt, nwaves, (int)tps, s_ctx};
}

int verify_max_rows() { return 8 * 3 * 16; }

// Workspace: running state first (fixed offsets for every call of one
// verification), then this call's split partials.
static size_t run_bytes(const vc_attn_shape& sh, size_t R) {
  const size_t units = (size_t)sh.batch * sh.n_kv_heads;
  return align_up(units * R * sh.head_dim * 4, 256) + align_up(units * R * 2 * 4, 256);
}
static size_t part_bytes(const vc_attn_shape& sh, size_t R, size_t S) {
  const size_t units = (size_t)sh.batch * sh.n_kv_heads;
  return align_up(units * S * R * sh.head_dim * 4, 256) + align_up(units * S * R * 2 * 4, 256);
}

size_t verify_ws_bytes(const vc_attn_shape& sh, int n_rows, int max_chunk_tokens) {
  const VerifyPlan p = verify_plan(sh, n_rows, max_chunk_tokens);
  const size_t R = (size_t)n_rows * (sh.n_q_heads / sh.n_kv_heads);
  return run_bytes(sh, R) + part_bytes(sh, R, (size_t)p.s_ctx + 1);
}

vc_status verify_launch(const vc_attn_shape& sh, int n_rows, const void* q, const void* k_new, const void* v_new,
                        const vc_kv_chunk& ctx, const int32_t* ctx_len, int flags, float* out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  const VerifyPlan plan = verify_plan(sh, n_rows, ctx.tok_count);
  VerifyParams P{};
  const size_t R = (size_t)n_rows * (sh.n_q_heads / sh.n_kv_heads);
  const size_t units = (size_t)sh.batch * sh.n_kv_heads;
  const size_t S = (size_t)plan.s_ctx + ((flags & VC_VERIFY_END) ? 1 : 0);
  char* w = static_cast<char*>(ws);
  P.run_o = reinterpret_cast<float*>(w);
  w += align_up(units * R * sh.head_dim * 4, 256);
  P.run_ml = reinterpret_cast<float*>(w);
  w += align_up(units * R * 2 * 4, 256);
  P.part_o = reinterpret_cast<float*>(w);
  w += align_up(units * S * R * sh.head_dim * 4, 256);
  P.part_ml = reinterpret_cast<float*>(w);
  P.q = static_cast<const uint16_t*>(q);
  P.k_new = static_cast<const uint16_t*>(k_new);
  P.v_new = static_cast<const uint16_t*>(v_new);
  P.ck = static_cast<const uint16_t*>(ctx.k);
  P.cv = static_cast<const uint16_t*>(ctx.v);
  P.t_cap = ctx.t_cap;
  P.tok_begin = ctx.tok_begin;
  P.tok_count = ctx.tok_count;
  P.ctx_len = ctx_len;
  P.out = out;
  P.B = sh.batch;
  P.Hq = sh.n_q_heads;
  P.Hkv = sh.n_kv_heads;
  P.g = sh.n_q_heads / sh.n_kv_heads;
  P.NR = n_rows;
  P.R = (int)R;
  P.tps = plan.tps;
  P.S_ctx = plan.s_ctx;
  P.S = (int)S;
  P.flags = flags;
  P.qscale = kLog2e / sqrtf((float)sh.head_dim);
  const dim3 grid(P.S, sh.n_kv_heads, sh.batch);
  if (sh.head_dim == 128) launch_verify<128>(P, plan.rt, plan.nwaves, grid, stream);
  else launch_verify<64>(P, plan.rt, plan.nwaves, grid, stream);
  vc_status st = check_launch("verify attention");
  if (st != VC_OK) return st;
  const dim3 mgrid((unsigned)R, sh.n_kv_heads, sh.batch);
  if (sh.head_dim == 128) hipLaunchKernelGGL((verify_merge_kernel<128>), mgrid, dim3(128), 0, stream, P);
  else hipLaunchKernelGGL((verify_merge_kernel<64>), mgrid, dim3(64), 0, stream, P);
  return check_launch("verify merge");
}

}  // namespace vc
