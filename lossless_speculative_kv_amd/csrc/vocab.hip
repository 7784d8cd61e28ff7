// Vocabulary projection with a fused greedy argmax (VeriCache summary, "Core
// algorithm" and "Experimental results": drafting and verification both pick
// tokens greedily; "P1": drafting also streams the model weights from HBM).
//
// logits[m][n] = sum_k bf16(h[m][k]) * W[n][k], fp32 accumulation on
// v_mfma_f32_16x16x32_bf16 with A = 16 vocabulary rows of W and B = 16 hidden
// rows. Contraction slots are permuted so that one load instruction reads 64
// contiguous bytes of each of 16 rows (the four lane groups take consecutive
// 16-byte pieces): lane group qg takes k = k0 + 32*kk + 8*qg + s in K-step kk
// (the B operand uses the same permutation).
//
// Three kernels share the epilogue:
//  * vocab_stream: M <= 16*MS rows (draft steps). Each wave owns 16*NA vocab
//    rows; W goes straight from HBM to registers, h (tiny) from L2: fp32
//    rounded to bf16 in registers for one m-tile, else the bf16 copy.
//    A workgroup of 8 waves fills a CU and its waves are paced.
//  * vocab_ring: 33 <= M <= 416 (verification). 8 waves = 4 vocab groups x
//    2 row groups; W and hidden rows pass through an LDS ring of
//    direct-to-LDS loads that every wave issues its share of.
//  * vocab_staged: M above 416. Each wave owns 32 vocab rows and all M rows; the
//    hidden rows are staged in LDS in 32-wide k chunks (double-buffered) and
//    shared by the 8 waves of the workgroup, so W is read from HBM exactly
//    once. Up to 18 row tiles the loads run ahead: the next W chunk and the
//    hidden chunk after it are in registers while the current one is
//    multiplied.
// Argmax: each workgroup reduces (logit, index) to one 64-bit key per row,
// key = ordered(logit) << 32 | ~index, whose maximum is the largest logit with
// the lowest index (-0 is folded to +0); a second kernel takes the max over
// workgroups. The result does not depend on scheduling.
#include "vc_internal.h"

namespace vc {

namespace {

struct VocabParams {
  const float* h;     // fp32 [M][K]
  uint16_t* hb;       // bf16 [Mp][K] (workspace)
  const uint16_t* w;  // bf16 [V][K]
  uint64_t* keys;     // [nwg][M] (workspace)
  int32_t* argmax;    // [M]
  float* max_logit;   // [M] or null
  float* logits;      // [M][V] or null
  int M, Mp, K, V, nwg;
  int hb_sliced;  // hb layout: 0 row-major [Mp][K]; 1 k-slice-major [K/32][Mp][32]
};

__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0) u = 0;  // -0 -> +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)idx);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(~(uint32_t)k); }

__device__ __forceinline__ uint64_t max_q_u64(uint64_t x) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  uint64_t k0 = ((uint64_t)b[0] << 32) | a[0], k1 = ((uint64_t)b[1] << 32) | a[1];
  x = k0 > k1 ? k0 : k1;
  lo = (uint32_t)x;
  hi = (uint32_t)(x >> 32);
  a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  k0 = ((uint64_t)b[0] << 32) | a[0];
  k1 = ((uint64_t)b[1] << 32) | a[1];
  return k0 > k1 ? k0 : k1;
}

// h fp32 -> bf16 (nearest even), rows M..Mp-1 zero; row-major, or
// k-slice-major (each 32-wide k slice of all rows contiguous) for the ring
// kernel, whose every stage then reads one contiguous block of hidden rows.
__global__ __launch_bounds__(256) void hidden_to_bf16_kernel(const VocabParams P) {
  const size_t n = (size_t)P.Mp * P.K;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t m = i / P.K, k = i % P.K;
    const uint16_t v = (m < (size_t)P.M) ? (uint16_t)f32_to_bf16_bits(P.h[i]) : (uint16_t)0;
    const size_t dst = P.hb_sliced ? ((k / 32) * P.Mp + m) * 32 + k % 32 : i;
    P.hb[dst] = v;
  }
}

// Reduce the per-wave candidates (vocab tile a, m-tile mt) into keys per row
// and write the optional logits. acc[a][mt][r]: logit of vocab row
// vbase + 16*a + 4*qg + r and hidden row 16*mt_row + n.
template <int NA, int NMT>
__device__ __forceinline__ void epilogue(const VocabParams& P, const f32x4 (&acc)[NA][NMT], int vbase,
                                         const int (&mrow)[NMT], int lane, uint64_t (&best)[NMT]) {
  const int n = lane & 15, qg = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int m = mrow[mt] + n;
    uint64_t bk = 0;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = vbase + 16 * a + 4 * qg + r;
        if (v < P.V) {
          const uint64_t k = make_key(acc[a][mt][r], v);
          bk = k > bk ? k : bk;
        }
      }
    best[mt] = max_q_u64(bk);
    if (P.logits != nullptr && m < P.M) {
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const int v0 = vbase + 16 * a + 4 * qg;
        float* dst = P.logits + (size_t)m * P.V + v0;
        if (v0 + 3 < P.V && (P.V & 3) == 0) {
          *reinterpret_cast<f32x4*>(dst) = acc[a][mt];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (v0 + r < P.V) dst[r] = acc[a][mt][r];
        }
      }
    }
  }
}

// Stream kernel: 8 waves x 64 vocab rows. Its registers hold two waves per
// SIMD, so a workgroup fills a CU (a CU with two workgroups would serve the
// older first and finish the younger late) and the waves are paced.
constexpr int kStreamWaves = 8;

// NA vocab tiles of 16 rows per wave (the plan picks NA per vocabulary size
// so that the workgroups fill the CUs in as few rounds as possible).
template <int MS, int NA>
__global__ __launch_bounds__(64 * kStreamWaves, 2) void vocab_stream_kernel(const VocabParams P) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const int vbase = (blockIdx.x * kStreamWaves + wave) * 16 * NA;
  __shared__ __attribute__((aligned(16))) int progress[8];  // k-steps of 256 each wave has started
  if (threadIdx.x < 8) progress[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prog_lds = lds_addr(progress);
  f32x4 acc[NA][MS];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < MS; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wrow[NA];
  bool wok[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int v = vbase + 16 * a + n;
    wok[a] = v < P.V;
    wrow[a] = P.w + (size_t)(wok[a] ? v : 0) * P.K + 8 * qg;
  }
  // With one m-tile the hidden rows are read as fp32 (L2 hits: every wave
  // reads them) and rounded to bf16 (nearest even) in registers; a row past
  // M reads row M - 1 and only feeds keys and logits that are never written.
  // Two m-tiles read the bf16 copy (the fp32 registers would spill).
  constexpr bool kRound = MS == 1;
  using HRaw = std::conditional_t<kRound, f32x4[MS][4][2], u32x4[MS][4]>;
  const float* hrow[MS];
  const uint16_t* hrow16[MS];
#pragma unroll
  for (int t = 0; t < MS; ++t) {
    hrow[t] = P.h + (size_t)min(16 * t + n, P.M - 1) * P.K + 8 * qg;
    hrow16[t] = P.hb + (size_t)(16 * t + n) * P.K + 8 * qg;
  }

  // W k-steps of 128 are double-buffered in registers: the loads of step
  // i + 1 are in flight while step i is multiplied. Every W load is
  // unconditional: a row past the vocabulary reads row 0 and only feeds
  // logits the epilogue skips (a load under a per-lane condition, or masked
  // right after it, is waited for at once). A step's hidden operands are
  // loaded just before the next step's W: vector-memory loads complete in
  // issue order, so waiting for the hidden values leaves the W loads in
  // flight.
  auto load = [&](u32x4 (&A)[NA][4], int k0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) A[a][kk] = *reinterpret_cast<const u32x4*>(wrow[a] + k0 + 32 * kk);
  };
  auto load_h = [&](HRaw& H, int k0) {
#pragma unroll
    for (int t = 0; t < MS; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if constexpr (kRound) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            H[t][kk][j] = *reinterpret_cast<const f32x4*>(hrow[t] + k0 + 32 * kk + 4 * j);
        } else {
          H[t][kk] = *reinterpret_cast<const u32x4*>(hrow16[t] + k0 + 32 * kk);
        }
      }
  };
  auto to_bf16 = [&](const HRaw& H, u32x4 (&B)[MS][4]) {
#pragma unroll
    for (int t = 0; t < MS; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if constexpr (kRound) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            B[t][kk][2 * j] = f32_to_bf16_bits(H[t][kk][j][0]) | (f32_to_bf16_bits(H[t][kk][j][1]) << 16);
            B[t][kk][2 * j + 1] = f32_to_bf16_bits(H[t][kk][j][2]) | (f32_to_bf16_bits(H[t][kk][j][3]) << 16);
          }
        } else {
          B[t][kk] = H[t][kk];
        }
      }
  };
  auto compute = [&](const u32x4 (&A)[NA][4], const u32x4 (&B)[MS][4]) {
#pragma unroll
    for (int t = 0; t < MS; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int a = 0; a < NA; ++a) acc[a][t] = mfma_bf16(A[a][kk], B[t][kk], acc[a][t]);
  };
  u32x4 Aa[NA][4], Ab[NA][4], B[MS][4];
  HRaw H;
  // a wave past the last vocab row has nothing to stream (and must not lead
  // the pacing)
  if (vbase < P.V) {
    load(Aa, 0);
    int k0 = 0;
    // (the scheduling barriers keep the W loads issued before the hidden
    // values are converted: the scheduler would otherwise sink them past
    // the wait for the hidden loads)
    for (; k0 + 256 <= P.K; k0 += 256) {
      load_h(H, k0);
      load(Ab, k0 + 128);
      __builtin_amdgcn_sched_barrier(0);
      pace_waves<kStreamWaves>(prog_lds, wave, k0 >> 8);
      to_bf16(H, B);
      compute(Aa, B);
      load_h(H, k0 + 128);
      if (k0 + 256 < P.K) load(Aa, k0 + 256);
      __builtin_amdgcn_sched_barrier(0);
      to_bf16(H, B);
      compute(Ab, B);
    }
    if (k0 < P.K) {  // K / 128 odd: the last step's W is already loaded
      load_h(H, k0);
      to_bf16(H, B);
      compute(Aa, B);
    }
  }
  int mrow[MS];
#pragma unroll
  for (int t = 0; t < MS; ++t) mrow[t] = 16 * t;
  uint64_t best[MS];
  epilogue<NA, MS>(P, acc, vbase, mrow, lane, best);
  __shared__ uint64_t red[kStreamWaves][16 * MS];
#pragma unroll
  for (int t = 0; t < MS; ++t)
    if (qg == 0) red[wave][16 * t + n] = best[t];
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kStreamWaves) {
    uint64_t k = red[0][m];
#pragma unroll
    for (int w = 1; w < kStreamWaves; ++w) k = red[w][m] > k ? red[w][m] : k;
    P.keys[(size_t)blockIdx.x * P.M + m] = k;
  }
}

// Staged kernel: 8 waves x 32 vocab rows; all m-tiles (NMT >= ceil(M/16)).
constexpr int kStagedWaves = 8;
constexpr int kKC = 32;  // k per LDS stage (one MFMA K-step)

template <int NMT>
__global__ __launch_bounds__(512) void vocab_staged_kernel(const VocabParams P) {
  constexpr int NA = 2, HSTR = kKC + 8;  // halfs per staged hidden row (16-byte aligned, skewed)
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem_raw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, qg = lane >> 4;
  const int mtiles = P.Mp / 16;
  const int vbase = (blockIdx.x * kStagedWaves + wave) * 32;
  f32x4 acc[NA][NMT];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NMT; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wrow[NA];
  bool wok[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int v = vbase + 16 * a + n;
    wok[a] = v < P.V;
    wrow[a] = P.w + (size_t)(wok[a] ? v : 0) * P.K;
  }
  const int stage_halfs = P.Mp * HSTR;
  // cooperative copy of hidden chunk [Mp][kKC] into LDS buffer `buf`
  auto stage = [&](int k0, int buf) {
    uint16_t* dst = hs + buf * stage_halfs;
    const int chunks = P.Mp * (kKC / 8);
    for (int c = threadIdx.x; c < chunks; c += 64 * kStagedWaves) {
      const int m = c / (kKC / 8), x = c % (kKC / 8);
      *reinterpret_cast<u32x4*>(dst + m * HSTR + 8 * x) =
          *reinterpret_cast<const u32x4*>(P.hb + (size_t)m * P.K + k0 + 8 * x);
    }
  };
  // W for one chunk: lane group qg of K-step kk reads k0 + 32*kk + 8*qg (with the other lane
  // groups, 64 contiguous bytes of each row per instruction)
  constexpr int KS = kKC / 32;  // K-steps per chunk
  // (unconditional loads: a row past the vocabulary reads row 0 and only
  // feeds logits the epilogue skips; a load under a per-lane condition, or
  // masked right after it, is waited for at once)
  auto load_w = [&](u32x4 (&A)[NA][KS], int k0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) A[a][kk] = *reinterpret_cast<const u32x4*>(wrow[a] + k0 + 32 * kk + 8 * qg);
  };
  auto compute = [&](const u32x4 (&A)[NA][KS], const uint16_t* cur) {
#pragma unroll
    for (int t = 0; t < NMT; ++t) {
      if (t < mtiles) {
        const uint16_t* hr = cur + (16 * t + n) * HSTR + 8 * qg;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const u32x4 B = *reinterpret_cast<const u32x4*>(hr + 32 * kk);
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[a][t] = mfma_bf16(A[a][kk], B, acc[a][t]);
        }
      }
    }
  };
  const int nk = P.K / kKC;
  if constexpr (NMT <= 18) {
    // Pipelined: W chunks double-buffered in registers, and the hidden chunk
    // two ahead loaded into registers while the current one is multiplied,
    // then written to its LDS buffer one iteration later (so neither load's
    // latency sits between two barriers).
    constexpr int HPT = (16 * NMT * (kKC / 8) + 64 * kStagedWaves - 1) / (64 * kStagedWaves);
    u32x4 hreg[HPT];
    const int chunks = P.Mp * (kKC / 8);
    // (a slot past the chunk loads the chunk's last unit and is not stored)
    auto hload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int c = min((int)threadIdx.x + i * 64 * kStagedWaves, chunks - 1);
        const int m = c / (kKC / 8), x = c % (kKC / 8);
        hreg[i] = *reinterpret_cast<const u32x4*>(P.hb + (size_t)m * P.K + k0 + 8 * x);
      }
    };
    auto hstore = [&](int buf) {
      uint16_t* dst = hs + buf * stage_halfs;
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int c = threadIdx.x + i * 64 * kStagedWaves;
        const int m = c / (kKC / 8), x = c % (kKC / 8);
        if (c < chunks) *reinterpret_cast<u32x4*>(dst + m * HSTR + 8 * x) = hreg[i];
      }
    };
    // W chunks in three register sets, loaded two chunks ahead (one chunk
    // ahead left the kernel bound by the loads' latency)
    // The loads of a chunk go out hidden first, then W: waiting for a hidden
    // chunk one iteration later (vector-memory loads complete in issue
    // order) then leaves that chunk's W loads in flight.
    u32x4 Aa[NA][KS], Ab[NA][KS], Ac[NA][KS];
    hload(0);
    hstore(0);
    if (nk > 1) hload(kKC);
    load_w(Aa, 0);
    if (nk > 1) load_w(Ab, kKC);
    __syncthreads();
    // iteration kc: hidden kc + 1 -> LDS; hidden and W of kc + 2 issued; W of
    // kc + 1 still in flight
    auto iter = [&](const u32x4 (&Acur)[NA][KS], u32x4 (&Aload)[NA][KS], int kc) {
      if (kc + 1 < nk) hstore((kc + 1) & 1);
      if (kc + 2 < nk) {
        hload((kc + 2) * kKC);
        load_w(Aload, (kc + 2) * kKC);
      }
      compute(Acur, hs + (kc & 1) * stage_halfs);
      __syncthreads();
    };
    int kc = 0;
    for (; kc + 3 <= nk; kc += 3) {
      iter(Aa, Ac, kc);
      iter(Ab, Aa, kc + 1);
      iter(Ac, Ab, kc + 2);
    }
    if (kc < nk) iter(Aa, Ac, kc);
    if (kc + 1 < nk) iter(Ab, Aa, kc + 1);
  } else {
    stage(0, 0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
      u32x4 A[NA][KS];
      load_w(A, kc * kKC);
      if (kc + 1 < nk) stage((kc + 1) * kKC, (kc + 1) & 1);
      compute(A, hs + (kc & 1) * stage_halfs);
      __syncthreads();
    }
  }
  int mrow[NMT];
#pragma unroll
  for (int t = 0; t < NMT; ++t) mrow[t] = 16 * t;
  uint64_t best[NMT];
  epilogue<NA, NMT>(P, acc, vbase, mrow, lane, best);
  // cross-wave reduction through LDS (reuses the staging area)
  uint64_t* red = reinterpret_cast<uint64_t*>(smem_raw);
#pragma unroll
  for (int t = 0; t < NMT; ++t)
    if (qg == 0 && t < mtiles) red[wave * P.Mp + 16 * t + n] = best[t];
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kStagedWaves) {
    uint64_t k = red[m];
    for (int w = 1; w < kStagedWaves; ++w) k = red[w * P.Mp + m] > k ? red[w * P.Mp + m] : k;
    P.keys[(size_t)blockIdx.x * P.M + m] = k;
  }
}

// Tiled kernel (up to 18 row tiles): 8 waves = 2 row groups x 4 vocab
// groups; a workgroup covers 256 vocab rows and all rows of the hidden
// matrix. W and hidden rows move in 32-wide k slices through a 4-stage LDS
// ring of direct-to-LDS loads (1 KB each: 16 rows x 64 bytes), issued by all
// waves three stages ahead; one workgroup barrier per stage. Each wave
// multiplies its 4 vocab tiles by its NMT2 row tiles from LDS (A and B
// operands are 16-byte reads of one row each, conflict-free), so W is read
// from HBM once at full rate while the MFMA work per byte of LDS stays high.
// Switched off: on its first run (M = 33, three row tiles) this kernel made
// the GPU report an illegal memory access, and again after the reads of
// rows-less waves were removed; the cause is not found (every address it
// forms for that shape is in range, and its built loop reuses no register of
// an in-flight LDS read before the wait), so the plan never selects it: the
// ring kernel serves M 33 .. 416.
constexpr bool kTiledEnabled = false;
constexpr int kTiledWaves = 8;
constexpr int kTVG = 4;              // vocab groups of 64 rows
constexpr int kTRows = kTVG * 64;    // vocab rows per workgroup
constexpr int kTStages = 4;
constexpr int kTWBytes = kTRows * 64;  // W slice of a stage: 256 rows x 32 k (bf16)

template <int NMT2>
struct TiledGeo {
  static constexpr int HCH = 2 * NMT2;                               // hidden 1 KB chunks of a stage
  static constexpr int HPW = (HCH + kTiledWaves - 1) / kTiledWaves;  // hidden chunks issued per wave
  static constexpr int NI = 2 + HPW;                                 // loads per wave per stage
  static constexpr int SB = kTWBytes + HCH * 1024;                   // bytes per stage
};

__device__ __forceinline__ uint32_t lds_addr32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}
// 16-byte LDS read the compiler does not track (it would otherwise wait for
// every pending direct-to-LDS load before it); ordered by the ring's waits.
__device__ __forceinline__ u32x4 lds_read16(const char* p) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr32(p)) : "memory");
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int NMT2>
__global__ __launch_bounds__(512, 2) void vocab_tiled_kernel(const VocabParams P) {
  using G = TiledGeo<NMT2>;
  constexpr int NA = 4;
  __shared__ __attribute__((aligned(16))) char ring[kTStages * G::SB];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const int vg = wave % kTVG, mg = wave / kTVG;
  const int vwg = blockIdx.x * kTRows;
  const int mtiles = P.Mp / 16, hch = P.Mp / 16;  // valid hidden chunks per stage
  const bool active = mg * NMT2 < mtiles;           // this wave's row group holds rows
  const int nk = P.K / 32;
  // buffer resources: this workgroup's W rows, and the padded hidden rows
  const uint64_t wb = reinterpret_cast<uint64_t>(P.w + (size_t)vwg * P.K);
  const uint32_t wrows = (uint32_t)max(0, min(kTRows, P.V - vwg));
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(wb >> 32)) << 32) |
                              __builtin_amdgcn_readfirstlane((uint32_t)wb)),
      (short)0, (int)__builtin_amdgcn_readfirstlane(wrows * (uint32_t)P.K * 2u), 0x00020000);
  const uint64_t hbb = reinterpret_cast<uint64_t>(P.hb);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(hbb >> 32)) << 32) |
                              __builtin_amdgcn_readfirstlane((uint32_t)hbb)),
      (short)0, (int)__builtin_amdgcn_readfirstlane((uint32_t)P.Mp * (uint32_t)P.K * 2u), 0x00020000);
  // lane l of a 1 KB chunk: row 16c + l/4, 16-byte piece l%4 of the 64-byte k slice
  const int lrow = lane >> 2, lpiece = lane & 3;
  auto issue = [&](int st) {
    char* stage = ring + (st % kTStages) * G::SB;
    const int k0 = min(st, nk - 1) * 32;  // past the end: reload the last slice into an unused stage
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = wave + kTiledWaves * j;  // W chunks 0..15
      const int voff = ((16 * c + lrow) * P.K + k0) * 2 + 16 * lpiece;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(stage + c * 1024), 16,
                                               voff, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < G::HPW; ++j) {
      const int c = min(wave + kTiledWaves * j, hch - 1);  // beyond the rows: the last chunk again
      const int voff = ((16 * c + lrow) * P.K + k0) * 2 + 16 * lpiece;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rh, (__attribute__((address_space(3))) void*)(stage + kTWBytes + c * 1024), 16, voff, 0, 0, 0);
    }
  };
  f32x4 acc[NA][NMT2];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NMT2; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0);
  issue(1);
  issue(2);
  for (int st = 0; st < nk; ++st) {
    wait_vmcnt<2 * G::NI>();  // this wave's loads of stage st have landed
    __builtin_amdgcn_s_barrier();  // everyone's have, and stage st - 1 is read
    issue(st + 3);
    // The reads are asynchronous and the compiler does not know it: every
    // path that issues one waits for it (lgkmcnt(0)) before anything else can
    // be given its registers, so a wave without row tiles issues none.
    if (active) {
      const char* stage = ring + (st % kTStages) * G::SB;
      u32x4 A[NA], B[NMT2];
#pragma unroll
      for (int a = 0; a < NA; ++a) A[a] = lds_read16(stage + (64 * vg + 16 * a + n) * 64 + 16 * qg);
#pragma unroll
      for (int t = 0; t < NMT2; ++t)
        B[t] = (mg * NMT2 + t < mtiles) ? lds_read16(stage + kTWBytes + (16 * (mg * NMT2 + t) + n) * 64 + 16 * qg)
                                        : u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every read above has returned
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NMT2; ++t)
        if (mg * NMT2 + t < mtiles)
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[a][t] = mfma_bf16(A[a], B[t], acc[a][t]);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  int mrow[NMT2];
#pragma unroll
  for (int t = 0; t < NMT2; ++t) mrow[t] = 16 * (mg * NMT2 + t);
  uint64_t best[NMT2];
  epilogue<NA, NMT2>(P, acc, vwg + 64 * vg, mrow, lane, best);
  // reduce over the 4 vocab groups of each row through LDS (the ring is idle)
  uint64_t* red = reinterpret_cast<uint64_t*>(ring);  // [kTVG][Mp]
#pragma unroll
  for (int t = 0; t < NMT2; ++t)
    if (qg == 0 && mg * NMT2 + t < mtiles) red[vg * P.Mp + 16 * (mg * NMT2 + t) + n] = best[t];
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kTiledWaves) {
    uint64_t k = red[m];
#pragma unroll
    for (int w = 1; w < kTVG; ++w) k = red[w * P.Mp + m] > k ? red[w * P.Mp + m] : k;
    P.keys[(size_t)blockIdx.x * P.M + m] = k;
  }
}

// Ring kernel (up to 26 row tiles): the verification product, MFMA-bound at
// large M. 8 waves = 4 vocab groups of 64 rows x 2 row groups of NT row
// tiles; a workgroup covers 256 vocab rows and all Mp hidden rows, so each W
// row is read from HBM once, and W and the hidden rows move in 32-wide k
// slices through a ring of STAGES = AHEAD + 2 LDS stages. Every wave issues
// a fixed share of each stage's direct-to-LDS loads (1 KB each: 16 rows x
// 64 bytes), AHEAD stages ahead, waits for its share of the current stage
// and meets the others at a bare barrier. The loads are asm statements
// (the compiler does not count them as pending LDS writes, so it inserts no
// vmcnt(0) before the ring reads) and the ring is read with plain LDS loads
// (16 bytes per lane, one row per lane, XOR-swizzled pieces so that each
// eight lanes hit distinct banks). Per stage a wave multiplies its 4 vocab
// tiles by its NT row tiles: 4 + NT operand reads for 4 * NT MFMAs.
// A stage reads 64 bytes of each 128-byte line of a W row; the loads keep the
// default cache policy, so the line's other half is an L2 hit one stage
// later (with non-temporal W loads each line was fetched from HBM twice:
// M = 264 went 452 -> 366 us, M = 33 at K = 8192 535 -> 417 us). The hidden
// rows sit in a k-slice-major copy, so a stage's hidden part is one
// contiguous block.
constexpr int kRingWaves = 8;
constexpr int kRingRows = 256;  // vocab rows per workgroup
constexpr int kRingWch = 16;    // W chunks per stage

template <int NT>
struct RingGeo {
  static constexpr int HCH = 2 * NT;                          // hidden chunks per stage
  static constexpr int NCH = kRingWch + HCH;                  // chunks per stage
  static constexpr int PER = (NCH + kRingWaves - 1) / kRingWaves;  // loads per wave per stage
  static constexpr int SB = NCH * 1024;                       // bytes per stage
  static constexpr int AHEAD = NT <= 2 ? 4 : NT <= 5 ? 3 : NT <= 9 ? 2 : 1;
  static constexpr int STAGES = AHEAD + 2;
  static_assert(STAGES * SB <= 150 * 1024, "ring fits the LDS");
  static_assert(AHEAD * PER < 64, "vmcnt range");
};

// piece position of 16-byte piece p of a 64-byte row r in the ring
__device__ __forceinline__ int ring_piece(int r, int p) { return p ^ ((r >> 2) & 3); }

// One 1 KB direct-to-LDS load: lane l copies global bytes voff .. voff + 15
// of the buffer to LDS address m0 + 16 l (default cache policy). Written as
// an asm statement (see above); M0 is reserved to the compiler, so its value
// is put back.
__device__ __forceinline__ void ring_dma(const int (&rsrc)[4], uint32_t m0, int voff) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 r = {rsrc[0], rsrc[1], rsrc[2], rsrc[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(m0), "s"(r)
      : "memory");
}

template <int NT>
__global__ __launch_bounds__(64 * kRingWaves, 1) void vocab_ring_kernel(const VocabParams P) {
  using G = RingGeo<NT>;
  constexpr int NA = 4;
  __shared__ __attribute__((aligned(1024))) char ring[G::STAGES * G::SB];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const int vg = wave % 4, mg = wave / 4;
  const int vwg = blockIdx.x * kRingRows;
  const int mtiles = P.Mp / 16;
  const int nk = P.K / 32;
  const int mt0 = mg * NT;  // first row tile of this wave's row group
  // buffer descriptors (base, stride 0, extent in bytes, flags): this
  // workgroup's W rows (rows past the vocabulary read as zero) and the
  // padded bf16 hidden rows
  const uint64_t wb = reinterpret_cast<uint64_t>(P.w) + (uint64_t)vwg * (uint64_t)P.K * 2u;
  const uint32_t wrows = (uint32_t)min(kRingRows, P.V - vwg);
  const int rw[4] = {(int)__builtin_amdgcn_readfirstlane((uint32_t)wb),
                     (int)(__builtin_amdgcn_readfirstlane((uint32_t)(wb >> 32)) & 0xFFFFu),
                     (int)__builtin_amdgcn_readfirstlane(wrows * (uint32_t)P.K * 2u), 0x00020000};
  const uint64_t hb = reinterpret_cast<uint64_t>(P.hb);
  const int rh[4] = {(int)__builtin_amdgcn_readfirstlane((uint32_t)hb),
                     (int)(__builtin_amdgcn_readfirstlane((uint32_t)(hb >> 32)) & 0xFFFFu),
                     (int)__builtin_amdgcn_readfirstlane((uint32_t)P.Mp * (uint32_t)P.K * 2u), 0x00020000};
  // lane l of a chunk fills row 16c + l / 4 at piece position l % 4, i.e. the
  // global piece that the swizzle places there
  const int lrow = lane >> 2, lpos = lane & 3;
  const uint32_t ring0 = lds_addr(ring);
  // Hidden chunks past the row tiles (2 NT tiles allocated, Mp / 16 real)
  // would read the next slice's rows in the k-slice-major copy; they load the
  // last real chunk again instead (into their own, never-read stage rows).
  // this wave's share of stage s: chunks wave * PER + i (past the last chunk:
  // the last one again, same data to the same place); past the last stage
  // the last k slice is loaded again into a stage no step reads
  auto issue = [&](int s) {
    const uint32_t slot = ring0 + (uint32_t)((s % G::STAGES) * G::SB);
    const int k0 = min(s, nk - 1) * 32;
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      const int q = min(wave * G::PER + i, G::NCH - 1);  // wave-uniform
      const int hsrc = min(q - kRingWch, mtiles - 1);     // hidden chunk whose rows are read
      const int row = 16 * (q < kRingWch ? q : hsrc) + lrow;
      // W rows are row-major; the hidden copy is k-slice-major ([K/32][Mp][32])
      const int voff =
          (q < kRingWch ? (row * P.K + k0) * 2 : ((k0 / 32) * P.Mp + row) * 64) + 16 * ring_piece(row, lpos);
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + (uint32_t)q * 1024u);
      if (q < kRingWch) ring_dma(rw, m0, voff);
      else ring_dma(rh, m0, voff);
    }
  };
  f32x4 acc[NA][NT];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < G::AHEAD; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    issue(s + G::AHEAD);
    // this wave's share of stage s has landed; after the barrier everyone's
    // has, and nobody reads the stage that the loads just issued overwrite
    wait_vmcnt<G::AHEAD * G::PER>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* stage = ring + (s % G::STAGES) * G::SB;
    u32x4 A[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const int row = 64 * vg + 16 * a + n;
      A[a] = *reinterpret_cast<const u32x4*>(stage + row * 64 + 16 * ring_piece(row, qg));
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (mt0 + t < mtiles) {
        const int row = 16 * (mt0 + t) + n;  // hidden row = its row in the hidden part of the stage
        const u32x4 B = *reinterpret_cast<const u32x4*>(stage + kRingWch * 1024 + row * 64 + 16 * ring_piece(row, qg));
#pragma unroll
        for (int a = 0; a < NA; ++a) acc[a][t] = mfma_bf16(A[a], B, acc[a][t]);
      }
    }
  }
  wait_vmcnt<0>();  // nothing may land after the ring is reused below
  __syncthreads();
  int mrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) mrow[t] = 16 * (mt0 + t);
  uint64_t best[NT];
  epilogue<NA, NT>(P, acc, vwg + 64 * vg, mrow, lane, best);
  // reduce over the 4 vocab groups of each row through LDS (the ring is idle)
  uint64_t* red = reinterpret_cast<uint64_t*>(ring);  // [4][Mp]
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (qg == 0 && mt0 + t < mtiles) red[vg * P.Mp + 16 * (mt0 + t) + n] = best[t];
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kRingWaves) {
    uint64_t k = red[m];
#pragma unroll
    for (int w = 1; w < 4; ++w) k = red[w * P.Mp + m] > k ? red[w * P.Mp + m] : k;
    P.keys[(size_t)blockIdx.x * P.M + m] = k;
  }
}

__global__ __launch_bounds__(256) void vocab_reduce_kernel(const VocabParams P) {
  const int m = blockIdx.x;
  uint64_t k = 0;
  for (int i = threadIdx.x; i < P.nwg; i += 256) {
    const uint64_t x = P.keys[(size_t)i * P.M + m];
    k = x > k ? x : k;
  }
  __shared__ uint64_t red[256];
  red[threadIdx.x] = k;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = red[threadIdx.x + s] > red[threadIdx.x] ? red[threadIdx.x + s] : red[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    P.argmax[m] = key_index(red[0]);
    if (P.max_logit) P.max_logit[m] = key_value(red[0]);
  }
}

template <int NMT>
void launch_staged(const VocabParams& P, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const size_t lds = (size_t)2 * P.Mp * (kKC + 8) * 2;
  const size_t red = (size_t)kStagedWaves * P.Mp * 8;
  const size_t bytes = lds > red ? lds : red;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&vocab_staged_kernel<NMT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  launch_ev(vocab_staged_kernel<NMT>, dim3(P.nwg), dim3(64 * kStagedWaves), (uint32_t)bytes, s, start, stop, P);
}

}  // namespace

struct VocabPlan {
  bool stream;
  int ms;     // stream: m-tiles
  int na;     // stream: vocab tiles of 16 rows per wave
  int nmt;    // staged: m-tiles template bound
  int tiled;  // tiled: m-tiles per wave (0 = not tiled)
  int ring;   // ring: row tiles per row group (0 = not the ring kernel)
  int nwg;
  int Mp;
};

// Compute units the stream plan fills (MI355X).
constexpr long kVocabCUs = 256;

VocabPlan vocab_plan(int M, int K, int V) {
  (void)K;
  VocabPlan p{};
  p.Mp = (M + 15) / 16 * 16;
  const int mt = p.Mp / 16;
  if (mt <= 2) {
    p.stream = true;
    p.ms = mt;
    // vocab tiles per wave: the fewest rounds of workgroups over the 256 CUs
    // times the rows each wave streams (a vocabulary of 152064 rows takes 297
    // workgroups of 512 rows, two rounds, but 238 of 640 rows, one round);
    // five tiles only with one m-tile (registers); on a tie the larger tile
    // count (fewer workgroups) wins
    const int cand[4] = {5, 4, 2, 1};
    long best = -1;
    for (int na : cand) {
      if (na == 5 && mt != 1) continue;
      const long nwg = (V + 16L * na * kStreamWaves - 1) / (16L * na * kStreamWaves);
      const long cost = (nwg + kVocabCUs - 1) / kVocabCUs * na;
      if (best < 0 || cost < best) {
        best = cost;
        p.na = na;
        p.nwg = (int)nwg;
      }
    }
  } else if (kTiledEnabled && mt <= 18) {
    p.stream = false;
    p.tiled = mt <= 6 ? 3 : mt <= 12 ? 6 : 9;
    p.nwg = (V + kTRows - 1) / kTRows;
  } else if (mt <= 26) {
    // the two row groups of NT tiles cover every row tile
    p.stream = false;
    p.ring = mt <= 4 ? 2 : mt <= 10 ? 5 : mt <= 18 ? 9 : 13;
    p.nwg = (V + kRingRows - 1) / kRingRows;
  } else {
    p.stream = false;
    p.nmt = mt <= 4 ? 4 : mt <= 8 ? 8 : mt <= 12 ? 12 : mt <= 18 ? 18 : mt <= 24 ? 24 : 28;
    p.nwg = (V + 32 * kStagedWaves - 1) / (32 * kStagedWaves);
  }
  return p;
}

int vocab_max_rows() { return 28 * 16; }

size_t vocab_ws_bytes(int M, int K, int V) {
  const VocabPlan p = vocab_plan(M, K, V);
  return align_up((size_t)p.Mp * K * 2, 256) + align_up((size_t)p.nwg * M * 8, 256);
}

vc_status vocab_launch(int M, int K, int V, const float* h, const void* w, int32_t* argmax, float* max_logit,
                       float* logits, void* ws, hipStream_t stream) {
  const VocabPlan plan = vocab_plan(M, K, V);
  VocabParams P{};
  P.h = h;
  P.hb = static_cast<uint16_t*>(ws);
  P.keys = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + align_up((size_t)plan.Mp * K * 2, 256));
  P.w = static_cast<const uint16_t*>(w);
  P.argmax = argmax;
  P.max_logit = max_logit;
  P.logits = logits;
  P.M = M;
  P.Mp = plan.Mp;
  P.K = K;
  P.V = V;
  P.nwg = plan.nwg;
  P.hb_sliced = plan.ring ? 1 : 0;
  const Timing tm = take_timing();
  const bool main_only = tm.scope == VC_TIME_MAIN_KERNEL;
  hipEvent_t mstart = main_only ? tm.start : nullptr, mstop = main_only ? tm.stop : nullptr;
  // the stream kernel with one m-tile rounds the hidden rows itself; the
  // others read the bf16 copy
  const bool convert = !plan.stream || plan.ms != 1;
  if (convert) {
    const size_t n = (size_t)plan.Mp * K;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    launch_ev(hidden_to_bf16_kernel, dim3(blocks), dim3(256), 0, stream, main_only ? nullptr : tm.start, nullptr, P);
  }
  if (plan.stream) {
    const dim3 block(64 * kStreamWaves);
    hipEvent_t start = (main_only || convert) ? mstart : tm.start;
    const dim3 grid(plan.nwg);
    if (plan.ms == 1) {
      switch (plan.na) {
        case 1: launch_ev(vocab_stream_kernel<1, 1>, grid, block, 0, stream, start, mstop, P); break;
        case 2: launch_ev(vocab_stream_kernel<1, 2>, grid, block, 0, stream, start, mstop, P); break;
        case 4: launch_ev(vocab_stream_kernel<1, 4>, grid, block, 0, stream, start, mstop, P); break;
        default: launch_ev(vocab_stream_kernel<1, 5>, grid, block, 0, stream, start, mstop, P); break;
      }
    } else {
      switch (plan.na) {
        case 1: launch_ev(vocab_stream_kernel<2, 1>, grid, block, 0, stream, start, mstop, P); break;
        case 2: launch_ev(vocab_stream_kernel<2, 2>, grid, block, 0, stream, start, mstop, P); break;
        default: launch_ev(vocab_stream_kernel<2, 4>, grid, block, 0, stream, start, mstop, P); break;
      }
    }
  } else if (plan.ring) {
    const dim3 grid(plan.nwg), block(64 * kRingWaves);
    switch (plan.ring) {
      case 2: launch_ev(vocab_ring_kernel<2>, grid, block, 0, stream, mstart, mstop, P); break;
      case 5: launch_ev(vocab_ring_kernel<5>, grid, block, 0, stream, mstart, mstop, P); break;
      case 9: launch_ev(vocab_ring_kernel<9>, grid, block, 0, stream, mstart, mstop, P); break;
      default: launch_ev(vocab_ring_kernel<13>, grid, block, 0, stream, mstart, mstop, P); break;
    }
  } else if (plan.tiled) {
    const dim3 grid(plan.nwg), block(64 * kTiledWaves);
    if (plan.tiled == 3) launch_ev(vocab_tiled_kernel<3>, grid, block, 0, stream, mstart, mstop, P);
    else if (plan.tiled == 6) launch_ev(vocab_tiled_kernel<6>, grid, block, 0, stream, mstart, mstop, P);
    else launch_ev(vocab_tiled_kernel<9>, grid, block, 0, stream, mstart, mstop, P);
  } else {
    switch (plan.nmt) {
      case 4: launch_staged<4>(P, stream, mstart, mstop); break;
      case 8: launch_staged<8>(P, stream, mstart, mstop); break;
      case 12: launch_staged<12>(P, stream, mstart, mstop); break;
      case 18: launch_staged<18>(P, stream, mstart, mstop); break;
      case 24: launch_staged<24>(P, stream, mstart, mstop); break;
      default: launch_staged<28>(P, stream, mstart, mstop); break;
    }
  }
  vc_status st = check_launch("vocab projection");
  if (st != VC_OK) return st;
  launch_ev(vocab_reduce_kernel, dim3(M), dim3(256), 0, stream, nullptr, main_only ? nullptr : tm.stop, P);
  return check_launch("vocab argmax reduce");
}

}  // namespace vc
