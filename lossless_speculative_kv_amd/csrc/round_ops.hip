// Round bookkeeping and compressor builders:
//  * greedy acceptance (VeriCache summary, "Core algorithm": accept up to the
//    first mismatch, plus a bonus token when all drafts match);
//  * commit / restart from the last accepted token, including the KIVI
//    residual flush;
//  * KIVI-style min/max quantiser (keys per channel over 32 tokens, values
//    per token over 32 channels) writing the stored layout of include/vc.h;
//  * token-drop selection (top-n scores per KV head, ascending positions).
// The compressors sit behind one interface (VeriCache summary, "Architecture
// support").
#include "vc_internal.h"

namespace vc {

namespace {

// ------------------------------------------------------------ accept ----
// x, y, committed: position-major [k+1][B].
__global__ __launch_bounds__(64) void accept_kernel(int B, int k, const int32_t* x, const int32_t* y,
                                                    int32_t* n_accept, int32_t* next_token, int32_t* committed) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int m = k;
  for (int c0 = 0; c0 < k; c0 += 64) {
    const int j = c0 + lane;
    const bool mis = (j < k) && (x[(size_t)(j + 1) * B + b] != y[(size_t)j * B + b]);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(mis);
    if (bal != 0) {
      m = c0 + (int)__builtin_ctzll(bal);
      break;
    }
  }
  const int32_t nxt = y[(size_t)m * B + b];
  if (committed != nullptr) {
    for (int j = lane; j <= k; j += 64)
      committed[(size_t)j * B + b] = (j < m) ? x[(size_t)(j + 1) * B + b] : (j == m ? nxt : -1);
  }
  // all reads of x are done before next_token (which may alias x_0) is written
  __syncthreads();
  if (lane == 0) {
    n_accept[b] = m;
    next_token[b] = nxt;
  }
}

// ------------------------------------------------------- fp64 -> fp16 ----
// Round a finite double to the nearest binary16 (ties to even), as bits.
__device__ uint16_t f64_to_f16_bits(double x) {
  const double a = fabs(x);
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (a >= 65520.0) return sign | 0x7C00u;  // rounds to infinity
  int e;
  (void)frexp(a, &e);                      // a = f * 2^e, f in [0.5, 1)
  const int ex = e - 1 < -14 ? -14 : e - 1;  // unbiased exponent, subnormal floor
  const double ulp = ldexp(1.0, ex - 10);
  const double r = rint(a / ulp) * ulp;    // exact scaling, nearest-even rounding
  const _Float16 h = (_Float16)(float)r;   // r is representable: exact conversion
  return sign | (__builtin_bit_cast(uint16_t, h) & 0x7FFFu);
}
__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) { return (double)(float)__builtin_bit_cast(_Float16, b); }

// ---------------------------------------------------------- quantise ----
struct QuantParams {
  const uint16_t* src_k;  // [u][src_t_cap][D], bf16 or fp16
  const uint16_t* src_v;
  int src_fp16, src_t_cap;
  // per-sequence block plan: nblk and destination block; src rows start at 0
  const int32_t* nblk_dev;  // [B] or null -> nblk_const
  int nblk_const;
  const int32_t* dst_blk_dev;  // [B] body_len (tokens) or null -> 0
  const int32_t* skip;         // [B] nonzero -> skip sequence (or null)
  char* blocks;  // block records [u][body_cap/32][8*D*(BITS+1)]
  int Hkv, body_cap;
};

// Key scales: the smallest value with at most three significant bits that is
// >= x (then fp16; exact in fp16's normal range). A bf16 query value times
// such a scale needs at most 8 + 3 significant bits, so the draft kernel's
// fp16 fold of the scale into the query is exact; rounding up keeps every
// code in range.
__device__ __forceinline__ double round_up_3sig(double x) {
  if (!(x > 0.0)) return 0.0;
  int e;
  const double m = frexp(x, &e);  // x = m * 2^e, m in [0.5, 1)
  return ldexp(ceil(m * 8.0) / 8.0, e);
}

template <int D, int BITS>
__global__ __launch_bounds__(256) void kivi_quantize_kernel(const QuantParams P) {
  constexpr int NG = D / 32, WPT = D * BITS / 32, VWL = D * BITS / 64, QMAX = (1 << BITS) - 1;
  const int x = blockIdx.x, hk = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  if (P.skip && P.skip[b]) return;
  const int nblk = P.nblk_dev ? P.nblk_dev[b] : P.nblk_const;
  if (x >= nblk) return;
  const int dblk = (P.dst_blk_dev ? P.dst_blk_dev[b] / 32 : 0) + x;
  const size_t unit = (size_t)b * P.Hkv + hk;
  __shared__ double vals_k[32][D + 1];
  __shared__ double vals_v[32][D + 1];
  __shared__ uint8_t ck[32][D];
  __shared__ uint8_t cv[32][D];
  __shared__ uint16_t sv_s[32][NG], sv_z[32][NG];
  for (int i = tid; i < 32 * D; i += 256) {
    const int t = i / D, d = i % D;
    const size_t off = (unit * P.src_t_cap + (size_t)x * 32 + t) * D + d;
    const uint16_t kb = P.src_k[off], vb = P.src_v[off];
    vals_k[t][d] = P.src_fp16 ? f16_bits_to_f64(kb) : (double)bf16_bits_to_f32(kb);
    vals_v[t][d] = P.src_fp16 ? f16_bits_to_f64(vb) : (double)bf16_bits_to_f32(vb);
  }
  __syncthreads();
  const size_t nbc = (size_t)P.body_cap / 32;
  // the block's record: key codes, value codes, key scale / zero, value scale / zero
  constexpr int KC = 0, VC = 4 * D * BITS, KS = 8 * D * BITS, VS = KS + 4 * D, REC = 8 * D * (BITS + 1);
  char* const rec = P.blocks + (unit * nbc + dblk) * REC;
  uint32_t* const rk = reinterpret_cast<uint32_t*>(rec + KC);
  uint32_t* const rv = reinterpret_cast<uint32_t*>(rec + VC);
  uint16_t* const rks = reinterpret_cast<uint16_t*>(rec + KS);  // scale [D], then zero [D] (run order)
  uint16_t* const rvs = reinterpret_cast<uint16_t*>(rec + VS);  // scale [D/32][32], then zero
  if (tid < D) {
    // keys: channel tid over 32 tokens
    const int d = tid;
    double mn = vals_k[0][d], mx = vals_k[0][d];
    for (int t = 1; t < 32; ++t) {
      mn = fmin(mn, vals_k[t][d]);
      mx = fmax(mx, vals_k[t][d]);
    }
    const uint16_t sb = f64_to_f16_bits(round_up_3sig((mx - mn) / (double)QMAX)), zb = f64_to_f16_bits(mn);
    const double sc = f16_bits_to_f64(sb), ze = f16_bits_to_f64(zb);
    for (int t = 0; t < 32; ++t) {
      double c = 0.0;
      if (sc != 0.0) c = fmin(fmax(rint((vals_k[t][d] - ze) / sc), 0.0), (double)QMAX);
      ck[t][d] = (uint8_t)c;
    }
    // key scale / zero in runs of 8 channels stored in the order 0, 2, 1, 3,
    // 4, 6, 5, 7 (the order of the draft kernel's code pairs)
    const int o = d & 7, pos = (d & ~7) | (4 * (o >> 2) + 2 * (o & 1) + ((o >> 1) & 1));
    rks[pos] = sb;
    rks[D + pos] = zb;
  } else if (tid < D + 32 * NG) {
    // values: token t, channel group j
    const int i = tid - D, t = i / NG, j = i % NG;
    double mn = vals_v[t][32 * j], mx = mn;
    for (int c = 1; c < 32; ++c) {
      mn = fmin(mn, vals_v[t][32 * j + c]);
      mx = fmax(mx, vals_v[t][32 * j + c]);
    }
    const uint16_t sb = f64_to_f16_bits((mx - mn) / (double)QMAX), zb = f64_to_f16_bits(mn);
    const double sc = f16_bits_to_f64(sb), ze = f16_bits_to_f64(zb);
    for (int c = 0; c < 32; ++c) {
      double q = 0.0;
      if (sc != 0.0) q = fmin(fmax(rint((vals_v[t][32 * j + c] - ze) / sc), 0.0), (double)QMAX);
      cv[t][32 * j + c] = (uint8_t)q;
    }
    sv_s[t][j] = sb;
    sv_z[t][j] = zb;
  }
  __syncthreads();
  // key words: token-major, natural channel packing
  for (int i = tid; i < 32 * WPT; i += 256) {
    const int t = i / WPT, w = i % WPT;
    uint32_t word = 0;
    constexpr int PER = 32 / BITS;
    for (int f = 0; f < PER; ++f) word |= (uint32_t)ck[t][w * PER + f] << (BITS * f);
    rk[t * WPT + w] = word;
  }
  // value words: lane L = 16q + c, word w covers m-tiles [w*4/BITS, (w+1)*4/BITS)
  for (int i = tid; i < 64 * VWL; i += 256) {
    const int L = i / VWL, w = i % VWL, q = L >> 4, c = L & 15;
    uint32_t word = 0;
    constexpr int MPW = 4 / BITS;
    for (int mm = 0; mm < MPW; ++mm) {
      const int m = w * MPW + mm;
      for (int s = 0; s < 8; ++s) {
        const int t = 4 * q + (s >> 1) + 16 * (s & 1);
        const int bit = (BITS == 2) ? 8 * (s >> 1) + 4 * (s & 1) + 2 * (m & 1)
                                    : 16 * (s >> 2) + 8 * (s & 1) + 4 * ((s >> 1) & 1);
        word |= (uint32_t)cv[t][16 * m + c] << bit;
      }
    }
    rv[L * VWL + w] = word;
  }
  for (int i = tid; i < NG * 32; i += 256) {
    const int j = i / 32, e = i % 32, q = e >> 3, s = e & 7;
    const int t = 4 * q + (s >> 1) + 16 * (s & 1);
    rvs[j * 32 + e] = sv_s[t][j];
    rvs[D + j * 32 + e] = sv_z[t][j];
  }
}

// ------------------------------------------------------------ commit ----
struct CommitParams {
  int B, Hkv, D, k, kind, residual;
  const int32_t* n_accept;
  const uint16_t* k_new;  // [k+1][B][Hkv][D]
  const uint16_t* v_new;
  uint16_t* full_k;  // [u][full_t_cap][D]
  uint16_t* full_v;
  int full_t_cap;
  int32_t* ctx_len;
  int32_t* body_len;
  int32_t* tail_len;
  int body_cap, tail_cap;
  uint16_t* tail_k;
  uint16_t* tail_v;
  int32_t* status;
};

struct SeqPlan {
  int m, ctx0, tail_start, new_tail, nf, ok;
};

__device__ __forceinline__ SeqPlan plan_seq(const CommitParams& P, int b) {
  SeqPlan s;
  s.m = P.n_accept[b];
  s.ctx0 = P.ctx_len[b];
  s.tail_start = (P.kind == VC_DRAFT_DENSE) ? 0 : P.tail_len[b] - P.k;
  s.new_tail = s.tail_start + s.m + 1;
  s.nf = 0;
  if (P.kind == VC_DRAFT_KIVI && s.new_tail - P.residual >= 32) s.nf = (s.new_tail - P.residual) / 32;
  bool ok = s.m >= 0 && s.m <= P.k && s.ctx0 + s.m + 1 <= P.full_t_cap;
  if (P.kind != VC_DRAFT_DENSE) ok = ok && s.tail_start >= 0 && s.new_tail <= P.tail_cap;
  if (P.kind == VC_DRAFT_KIVI) ok = ok && (P.body_len[b] + 32 * s.nf <= P.body_cap) && (P.body_len[b] % 32 == 0);
  s.ok = ok ? 1 : 0;
  return s;
}

// Append block rows 0..m to the full cache and rewrite them into the tail.
__global__ __launch_bounds__(64) void commit_rows_kernel(const CommitParams P) {
  const int i = blockIdx.x, hk = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const SeqPlan s = plan_seq(P, b);
  if (i == 0 && hk == 0 && t == 0) P.status[b] = s.ok ? 0 : 1;
  if (!s.ok || i > s.m) return;
  const int D = P.D, chunks = D / 8;
  if (t >= chunks) return;
  const size_t unit = (size_t)b * P.Hkv + hk;
  const size_t src = (((size_t)i * P.B + b) * P.Hkv + hk) * D + 8 * t;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(P.k_new + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(P.v_new + src);
  const size_t dst = (unit * P.full_t_cap + s.ctx0 + i) * D + 8 * t;
  *reinterpret_cast<u32x4*>(P.full_k + dst) = kv;
  *reinterpret_cast<u32x4*>(P.full_v + dst) = vv;
  if (P.kind == VC_DRAFT_DENSE) return;
  const size_t td = (unit * P.tail_cap + s.tail_start + i) * D + 8 * t;
  if (P.kind == VC_DRAFT_KIVI) {
    u32x4 ko, vo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ko[e] = pack_f16(bf16_bits_to_f32(kv[e] & 0xFFFFu), bf16_bits_to_f32(kv[e] >> 16));
      vo[e] = pack_f16(bf16_bits_to_f32(vv[e] & 0xFFFFu), bf16_bits_to_f32(vv[e] >> 16));
    }
    *reinterpret_cast<u32x4*>(P.tail_k + td) = ko;
    *reinterpret_cast<u32x4*>(P.tail_v + td) = vo;
  } else {
    *reinterpret_cast<u32x4*>(P.tail_k + td) = kv;
    *reinterpret_cast<u32x4*>(P.tail_v + td) = vv;
  }
}

// Per-sequence flush plan for the quantiser: number of 32-token blocks to
// move from the tail into the body (0 when not KIVI or not ok).
__global__ void commit_flush_plan_kernel(const CommitParams P, int32_t* nf_out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= P.B) return;
  const SeqPlan s = plan_seq(P, b);
  nf_out[b] = (P.status[b] == 0) ? s.nf : 0;
}

// Drop the flushed rows from the tail: rows [32nf, new_tail) move to [0, ...),
// in chunks of 32nf rows so that source and destination never overlap.
__global__ __launch_bounds__(256) void commit_shift_kernel(const CommitParams P, const int32_t* nf_dev) {
  const int hk = blockIdx.x, b = blockIdx.y;
  if (P.status[b] != 0) return;
  const SeqPlan s = plan_seq(P, b);
  const int nf = nf_dev[b];
  if (nf == 0) return;
  const int shift = 32 * nf, keep = s.new_tail - shift, D = P.D, chunks = D / 8;
  const size_t unit = (size_t)b * P.Hkv + hk;
  uint16_t* tk = P.tail_k + unit * P.tail_cap * D;
  uint16_t* tv = P.tail_v + unit * P.tail_cap * D;
  for (int r0 = 0; r0 < keep; r0 += shift) {
    const int rows = min(shift, keep - r0);
    for (int i = threadIdx.x; i < rows * chunks; i += 256) {
      const int r = r0 + i / chunks, c = i % chunks;
      *reinterpret_cast<u32x4*>(tk + (size_t)r * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(tk + (size_t)(r + shift) * D + 8 * c);
      *reinterpret_cast<u32x4*>(tv + (size_t)r * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(tv + (size_t)(r + shift) * D + 8 * c);
    }
    __syncthreads();
  }
}

__global__ void commit_lens_kernel(const CommitParams P, const int32_t* nf_dev) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= P.B || P.status[b] != 0) return;
  const SeqPlan s = plan_seq(P, b);
  const int nctx = s.ctx0 + s.m + 1;
  if (P.kind == VC_DRAFT_KIVI) {
    const int nf = nf_dev[b];
    P.tail_len[b] = s.new_tail - 32 * nf;
    P.body_len[b] = P.body_len[b] + 32 * nf;
  } else if (P.kind == VC_DRAFT_TOKDROP) {
    P.tail_len[b] = s.new_tail;
  } else {
    P.body_len[b] = nctx;
    P.tail_len[b] = 0;
  }
  P.ctx_len[b] = nctx;
}

// ------------------------------------------------------- token drop ----
__device__ __forceinline__ uint32_t ord32(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 1024;

// One workgroup per (sequence, KV head): radix-select the n_keep-th largest
// key, then a stable compaction keeps every larger key and the lowest-index
// ties, writing positions in ascending order.
__global__ __launch_bounds__(kSelThreads) void tokdrop_select_kernel(const float* scores, int T, int n_keep,
                                                                     int32_t* kept) {
  const size_t unit = blockIdx.x;
  const float* sc = scores + unit * (size_t)T;
  int32_t* out = kept + unit * (size_t)n_keep;
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_mask, sh_krem;
  __shared__ uint32_t scan_a[kSelThreads], scan_b[kSelThreads];
  if (tid == 0) {
    sh_prefix = 0;
    sh_mask = 0;
    sh_krem = (uint32_t)n_keep;
  }
  __syncthreads();
  if (n_keep <= 0) return;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh_prefix, mask = sh_mask;
    for (int i = tid; i < T; i += kSelThreads) {
      const uint32_t k = ord32(sc[i]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t krem = sh_krem, above = 0;
      int bin = 255;
      for (; bin >= 0; --bin) {
        if (above + hist[bin] >= krem) break;
        above += hist[bin];
      }
      sh_krem = krem - above;
      sh_prefix = prefix | ((uint32_t)bin << shift);
      sh_mask = mask | (0xFFu << shift);
    }
    __syncthreads();
  }
  const uint32_t thr = sh_prefix, ties_kept = sh_krem;
  // contiguous ranges per thread for a stable order
  const int per = (T + kSelThreads - 1) / kSelThreads;
  const int i0 = min(T, tid * per), i1 = min(T, i0 + per);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = ord32(sc[i]);
    gt += k > thr;
    eq += k == thr;
  }
  // exclusive scan of eq (ties before this range)
  scan_a[tid] = eq;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const uint32_t v = tid >= off ? scan_a[tid - off] : 0u;
    __syncthreads();
    scan_a[tid] += v;
    __syncthreads();
  }
  const uint32_t eq_before = scan_a[tid] - eq;
  const uint32_t eq_take = eq_before >= ties_kept ? 0u : min(eq, ties_kept - eq_before);
  const uint32_t mine = gt + eq_take;
  scan_b[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const uint32_t v = tid >= off ? scan_b[tid - off] : 0u;
    __syncthreads();
    scan_b[tid] += v;
    __syncthreads();
  }
  uint32_t pos = scan_b[tid] - mine;
  uint32_t taken_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = ord32(sc[i]);
    bool keep = k > thr;
    if (k == thr && taken_eq < eq_take) {
      keep = true;
      ++taken_eq;
    }
    if (keep) out[pos++] = i;
  }
}

// Rows [row0, row0 + n) of bf16 src -> fp16 tail rows [0, n).
__global__ void tail_from_rows_kernel(const uint16_t* src_k, const uint16_t* src_v, int src_t_cap, int row0, int n,
                                      int D, int tail_cap, uint16_t* tail_k, uint16_t* tail_v) {
  const size_t unit = blockIdx.y;
  const int chunks = D / 8;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n * chunks; i += gridDim.x * blockDim.x) {
    const int r = i / chunks, c = i % chunks;
    const size_t s = (unit * src_t_cap + row0 + r) * D + 8 * c, d = (unit * tail_cap + r) * D + 8 * c;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(src_k + s), vv = *reinterpret_cast<const u32x4*>(src_v + s);
    u32x4 ko, vo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ko[e] = pack_f16(bf16_bits_to_f32(kv[e] & 0xFFFFu), bf16_bits_to_f32(kv[e] >> 16));
      vo[e] = pack_f16(bf16_bits_to_f32(vv[e] & 0xFFFFu), bf16_bits_to_f32(vv[e] >> 16));
    }
    *reinterpret_cast<u32x4*>(tail_k + d) = ko;
    *reinterpret_cast<u32x4*>(tail_v + d) = vo;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

}  // namespace

vc_status fill_i32_launch(int32_t* p, int n, int32_t value, hipStream_t stream) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n, value);
  return check_launch("fill");
}

vc_status tail_from_rows_launch(const vc_attn_shape& sh, const void* src_k, const void* src_v, int src_t_cap,
                                int row0, int n, const vc_draft_cache& dc, hipStream_t stream) {
  if (n <= 0) return VC_OK;
  const int chunks = n * sh.head_dim / 8;
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)(sh.batch * sh.n_kv_heads));
  hipLaunchKernelGGL(tail_from_rows_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(src_k),
                     static_cast<const uint16_t*>(src_v), src_t_cap, row0, n, sh.head_dim, dc.tail_cap,
                     static_cast<uint16_t*>(dc.tail_k), static_cast<uint16_t*>(dc.tail_v));
  return check_launch("kivi tail");
}

vc_status accept_launch(int B, int k, const int32_t* x, const int32_t* y, int32_t* n_accept, int32_t* next_token,
                        int32_t* committed, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, stream, B, k, x, y, n_accept, next_token, committed);
  return check_launch("greedy accept");
}

vc_status kivi_quantize_launch(const vc_attn_shape& sh, int bits, const void* src_k, const void* src_v, int src_fp16,
                               int src_t_cap, int grid_blocks, int nblk_const, const int32_t* nblk_dev,
                               const int32_t* dst_tok_dev, const int32_t* skip, const vc_draft_cache& dc,
                               hipStream_t stream) {
  QuantParams P{};
  P.src_k = static_cast<const uint16_t*>(src_k);
  P.src_v = static_cast<const uint16_t*>(src_v);
  P.src_fp16 = src_fp16;
  P.src_t_cap = src_t_cap;
  P.nblk_dev = nblk_dev;
  P.nblk_const = nblk_const;
  P.dst_blk_dev = dst_tok_dev;
  P.skip = skip;
  P.blocks = static_cast<char*>(dc.kivi_blocks);
  P.Hkv = sh.n_kv_heads;
  P.body_cap = dc.body_cap;
  if (grid_blocks <= 0) return VC_OK;
  const dim3 grid(grid_blocks, sh.n_kv_heads, sh.batch);
  if (sh.head_dim == 128 && bits == 2) hipLaunchKernelGGL((kivi_quantize_kernel<128, 2>), grid, dim3(256), 0, stream, P);
  else if (sh.head_dim == 128) hipLaunchKernelGGL((kivi_quantize_kernel<128, 4>), grid, dim3(256), 0, stream, P);
  else if (bits == 2) hipLaunchKernelGGL((kivi_quantize_kernel<64, 2>), grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL((kivi_quantize_kernel<64, 4>), grid, dim3(256), 0, stream, P);
  return check_launch("kivi quantize");
}

vc_status commit_launch(const vc_attn_shape& sh, int k, const int32_t* n_accept, const void* k_new,
                        const void* v_new, void* full_k, void* full_v, int full_t_cap, int32_t* ctx_len,
                        const vc_draft_cache& dc, int32_t* status, int32_t* scratch_nf, hipStream_t stream) {
  CommitParams P{};
  P.B = sh.batch;
  P.Hkv = sh.n_kv_heads;
  P.D = sh.head_dim;
  P.k = k;
  P.kind = dc.kind;
  P.residual = dc.residual;
  P.n_accept = n_accept;
  P.k_new = static_cast<const uint16_t*>(k_new);
  P.v_new = static_cast<const uint16_t*>(v_new);
  P.full_k = static_cast<uint16_t*>(full_k);
  P.full_v = static_cast<uint16_t*>(full_v);
  P.full_t_cap = full_t_cap;
  P.ctx_len = ctx_len;
  P.body_len = dc.body_len;
  P.tail_len = dc.tail_len;
  P.body_cap = dc.body_cap;
  P.tail_cap = dc.tail_cap;
  P.tail_k = static_cast<uint16_t*>(dc.tail_k);
  P.tail_v = static_cast<uint16_t*>(dc.tail_v);
  P.status = status;
  hipLaunchKernelGGL(commit_rows_kernel, dim3(k + 1, sh.n_kv_heads, sh.batch), dim3(64), 0, stream, P);
  vc_status st = check_launch("commit rows");
  if (st != VC_OK) return st;
  const unsigned bb = (unsigned)((sh.batch + 255) / 256);
  hipLaunchKernelGGL(commit_flush_plan_kernel, dim3(bb), dim3(256), 0, stream, P, scratch_nf);
  if ((st = check_launch("commit plan")) != VC_OK) return st;
  if (dc.kind == VC_DRAFT_KIVI) {
    st = kivi_quantize_launch(sh, dc.bits, dc.tail_k, dc.tail_v, 1, dc.tail_cap, dc.tail_cap / 32, 0, scratch_nf,
                              dc.body_len, status, dc, stream);
    if (st != VC_OK) return st;
    hipLaunchKernelGGL(commit_shift_kernel, dim3(sh.n_kv_heads, sh.batch), dim3(256), 0, stream, P,
                       (const int32_t*)scratch_nf);
    if ((st = check_launch("commit shift")) != VC_OK) return st;
  }
  hipLaunchKernelGGL(commit_lens_kernel, dim3(bb), dim3(256), 0, stream, P, (const int32_t*)scratch_nf);
  return check_launch("commit lengths");
}

vc_status tokdrop_launch(const vc_attn_shape& sh, const float* scores, int T, int n_keep, int32_t* kept,
                         hipStream_t stream) {
  hipLaunchKernelGGL(tokdrop_select_kernel, dim3(sh.batch * sh.n_kv_heads), dim3(kSelThreads), 0, stream, scores, T,
                     n_keep, kept);
  return check_launch("token-drop select");
}

}  // namespace vc
