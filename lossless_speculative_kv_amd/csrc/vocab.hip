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
// Two kernels share the epilogue:
//  * vocab_stream: M <= 32 rows (draft steps). Each workgroup takes an equal
//    share of the vocabulary tiles (one per CU), each wave up to NA tiles of
//    16 rows; W goes straight from HBM to registers, h (tiny) from L2: fp32
//    rounded to bf16 in registers up to 8 rows, else the bf16 copy. A
//    workgroup of 8 waves fills a CU and its waves are paced.
//  * vocab_ring: 33 <= M <= 448 (verification). 8 waves = VG vocab groups x
//    8 / VG row groups; W and hidden rows pass through an LDS ring of
//    direct-to-LDS loads that every wave issues its share of.
// (A third, switched-off kernel is kept below: vocab_tiled.)
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
  uint64_t* keys;     // [nwg key slots][M] (workspace)
  int32_t* argmax;    // [M]
  float* max_logit;   // [M] or null
  float* logits;      // [M][V] or null
  int M, Mp, K, V, nwg;
  int hb_sliced;  // hb layout: 0 row-major [Mp][K]; 1 k-slice-major [K/32][Mp][32]
  // ring kernel: slices [0, full) are done whole, each later one in `split`
  // parts of the k range whose products go to `part` (workspace,
  // [part][wave][4][NT][64 lanes] f32x4) for vocab_fixup_kernel
  float* part;
  int full, split;
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
// (sink(mt, key): the wave's best of row mrow[mt] + lane % 16, in every lane of
// the row) and write the optional logits. acc[a][mt][r]: logit of vocab row
// vbase + 16*a + 4*qg + r and hidden row 16*mt_row + n; vocab rows from vlim
// on (past the vocabulary, or past the caller's share of it) are skipped.
template <int NA, int NMT, typename Sink>
__device__ __forceinline__ void epilogue(const VocabParams& P, const f32x4 (&acc)[NA][NMT], int vbase,
                                         const int (&mrow)[NMT], int lane, int vlim, const Sink& sink) {
  const int n = lane & 15, qg = lane >> 4;
  // every vocab row of the wave below vlim (all workgroups but the last): the
  // lane's best is a plain float maximum in increasing index order, the first
  // index kept among equal values (-0 == +0; NaN never compares greater), and
  // becomes a key once per row tile; otherwise each element is tested
  const bool whole = vbase + 16 * NA <= vlim;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int m = mrow[mt] + n;
    uint64_t bk = 0;
    if (whole) {
      float bx = -__builtin_huge_valf();
      int bi = vbase + 4 * qg;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[a][mt][r];
          const bool gt = x > bx;
          bx = gt ? x : bx;
          bi = gt ? vbase + 16 * a + 4 * qg + r : bi;
        }
      bk = make_key(bx, bi);
    } else {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = vbase + 16 * a + 4 * qg + r;
          if (v < vlim) {
            const uint64_t k = make_key(acc[a][mt][r], v);
            bk = k > bk ? k : bk;
          }
        }
    }
    sink(mt, max_q_u64(bk));
    if (P.logits != nullptr && m < P.M) {
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const int v0 = vbase + 16 * a + 4 * qg;
        float* dst = P.logits + (size_t)m * P.V + v0;
        if (v0 + 3 < vlim && (P.V & 3) == 0) {
          *reinterpret_cast<f32x4*>(dst) = acc[a][mt];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (v0 + r < vlim) dst[r] = acc[a][mt][r];
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
template <int MS, int NA, bool ROUND>
__global__ __launch_bounds__(64 * kStreamWaves, 2) void vocab_stream_kernel(const VocabParams P) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  // this workgroup's share of the vocabulary tiles of 16 rows: tiles
  // [t_lo, t_hi), an equal share (within one tile) of every workgroup's, so
  // the grid can match the compute units; wave w takes NA of them from
  // t_lo + NA w (slots past t_hi load tile t_hi - 1 again, an L2 hit, and
  // store nothing)
  const long ntv = (P.V + 15) / 16;
  const int t_lo = (int)(blockIdx.x * ntv / gridDim.x), t_hi = (int)((blockIdx.x + 1) * ntv / gridDim.x);
  const int tfirst = t_lo + wave * NA;
  const int vbase = tfirst * 16;
  const int vlim = min(P.V, t_hi * 16);
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
    const int v = min(tfirst + a, t_hi - 1) * 16 + n;
    wok[a] = v < P.V;
    wrow[a] = P.w + (size_t)(wok[a] ? v : 0) * P.K + 8 * qg;
  }
  // ROUND (one m-tile, at most 8 rows): the hidden rows are read as fp32
  // (L2 hits: every wave reads them) and rounded to bf16 (nearest even) in
  // registers, which saves the conversion kernel; a row past M reads row
  // M - 1 and only feeds keys and logits that are never written. Otherwise
  // the bf16 copy is read: half the bytes of fp32 per wave, which at 16 rows
  // is worth the conversion (Qwen-32B draft step, M = 16: 309 -> 283 us) and
  // with two m-tiles keeps the registers from spilling.
  static_assert(!ROUND || MS == 1, "rounding in registers with one m-tile");
  constexpr bool kRound = ROUND;
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
  // a wave past its workgroup's share has nothing to stream (and must not
  // lead the pacing)
  if (tfirst < t_hi) {
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
  epilogue<NA, MS>(P, acc, vbase, mrow, lane, vlim, [&](int t, uint64_t k) { best[t] = k; });
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
// ring kernel serves M 33 .. 448.
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
  epilogue<NA, NMT2>(P, acc, vwg + 64 * vg, mrow, lane, P.V, [&](int t, uint64_t k) { best[t] = k; });
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

// Ring kernel (up to 28 row tiles): the verification product, MFMA-bound at
// large M. 8 waves = VG vocab groups of 64 rows x 8 / VG row groups of NT
// row tiles; a workgroup covers 64 VG vocab rows and all Mp hidden rows, so
// each W row is read from HBM once, and W and the hidden rows move in
// 32-wide k slices through a ring of STAGES = AHEAD + 1 LDS stages. Every
// wave issues a fixed share of each stage's direct-to-LDS loads (1 KB each:
// 16 rows x 64 bytes), AHEAD stages ahead: it waits for its share of the
// current stage, meets the others at a bare barrier and then issues the
// loads of stage s + AHEAD into the slot of stage s - 1, which everyone has
// finished reading (one stage more in flight than issuing before the
// barrier: M = 416 815 -> 779 us). The loads are asm statements
// (the compiler does not count them as pending LDS writes, so it inserts no
// vmcnt(0) before the ring reads) and the ring is read with plain LDS loads
// (16 bytes per lane, one row per lane, XOR-swizzled pieces so that each
// eight lanes hit distinct banks). Per stage a wave multiplies its 4 vocab
// tiles by its NT row tiles: 4 + NT operand reads for 4 * NT MFMAs.
// Counters (M = 416): 8 LDS-active cycles per 16-byte read instruction, half
// of them counted as bank conflicts, whatever the swizzle; MFMA busy 32%.
// A stage reads 64 bytes of each 128-byte line of a W row; the loads keep the
// default cache policy, so the line's other half is an L2 hit one stage
// later (with non-temporal W loads each line was fetched from HBM twice:
// M = 264 went 452 -> 366 us, M = 33 at K = 8192 535 -> 417 us). The hidden
// rows sit in a k-slice-major copy, so a stage's hidden part is one
// contiguous block. A workgroup fills a CU, so the slices run in rounds of
// the 256 CUs; when the last round would leave half of them or more idle,
// each of its slices is cut into parts of the k range that fill them, and
// vocab_fixup_kernel adds a slice's parts in part order and finishes it.
constexpr int kRingWaves = 8;
// VG vocab groups of 64 rows x (8 / VG) row groups of NT row tiles
template <int NT, int VG>
struct RingGeo {
  static constexpr int RG = kRingWaves / VG;                  // row groups
  static constexpr int ROWS = 64 * VG;                        // vocab rows per workgroup
  static constexpr int WCH = 4 * VG;                          // W chunks per stage
  static constexpr int HCH = RG * NT;                         // hidden chunks per stage
  static constexpr int NCH = WCH + HCH;                       // chunks per stage
  static constexpr int PER = (NCH + kRingWaves - 1) / kRingWaves;  // loads per wave per stage
  static constexpr int SB = NCH * 1024;                       // bytes per stage
  static constexpr int STAGES = (150 * 1024) / SB < 8 ? (150 * 1024) / SB : 8;
  static constexpr int AHEAD = STAGES - 1;
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

// The end of a slice (64 VG vocab rows, all hidden rows): the per-row best of
// each wave's products (epilogue), then the best over the VG vocab groups
// through LDS (lds: at least VG * Mp keys, free), stored as the slice's keys.
template <int NT, int VG>
__device__ __forceinline__ void ring_finish(const VocabParams& P, const f32x4 (&acc)[4][NT], int slice, char* lds,
                                            int lane, int wave) {
  using G = RingGeo<NT, VG>;
  const int n = lane & 15, qg = lane >> 4;
  const int vg = wave % VG, mg = wave / VG;
  const int mtiles = P.Mp / 16;
  const int mt0 = mg * NT;
  int mrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) mrow[t] = 16 * (mt0 + t);
  // each row tile's best goes to LDS as soon as it is known; then the best
  // over the VG vocab groups of each row
  uint64_t* red = reinterpret_cast<uint64_t*>(lds);  // [VG][Mp]
  epilogue<4, NT>(P, acc, slice * G::ROWS + 64 * vg, mrow, lane, P.V, [&](int t, uint64_t k) {
    if (qg == 0 && mt0 + t < mtiles) red[vg * P.Mp + 16 * (mt0 + t) + n] = k;
  });
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kRingWaves) {
    uint64_t k = red[m];
#pragma unroll
    for (int w = 1; w < VG; ++w) k = red[w * P.Mp + m] > k ? red[w * P.Mp + m] : k;
    P.keys[(size_t)slice * P.M + m] = k;
  }
}

template <int NT, int VG>
__global__ __launch_bounds__(64 * kRingWaves, 1) void vocab_ring_kernel(const VocabParams P) {
  using G = RingGeo<NT, VG>;
  constexpr int NA = 4;
  __shared__ __attribute__((aligned(1024))) char ring[G::STAGES * G::SB];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const int vg = wave % VG, mg = wave / VG;
  const int mtiles = P.Mp / 16;
  const int nk = P.K / 32;
  // this workgroup's slice and k slices [kb, ke): slices below P.full whole,
  // every later one in P.split parts (part >= 0: this workgroup's index
  // among the parts)
  int slice = blockIdx.x, kb = 0, ke = nk, part = -1;
  if ((int)blockIdx.x >= P.full) {
    const int j = blockIdx.x - P.full, pp = j % P.split;
    slice = P.full + j / P.split;
    kb = pp * nk / P.split;
    ke = (pp + 1) * nk / P.split;
    part = j;
  }
  const int vwg = slice * G::ROWS;
  const int mt0 = mg * NT;  // first row tile of this wave's row group
  // buffer descriptors (base, stride 0, extent in bytes, flags): this
  // workgroup's W rows (rows past the vocabulary read as zero) and the
  // padded bf16 hidden rows
  const uint64_t wb = reinterpret_cast<uint64_t>(P.w) + (uint64_t)vwg * (uint64_t)P.K * 2u;
  const uint32_t wrows = (uint32_t)min(G::ROWS, P.V - vwg);
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
  // this wave's share of stage s: chunks wave + 8 i (past the last chunk:
  // the last one again, same data to the same place); past the last stage
  // the last k slice is loaded again into a stage no step reads. The W
  // chunks are the first WCH, a multiple of the 8 waves, so whether a chunk
  // is W or hidden depends on i alone and the unrolled loop has no branch.
  static_assert(G::WCH % kRingWaves == 0, "W chunks dealt evenly");
  auto issue = [&](int s) {
    const uint32_t slot = ring0 + (uint32_t)((s % G::STAGES) * G::SB);
    const int k0 = min(s, ke - 1) * 32;
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      const int q = min(wave + kRingWaves * i, G::NCH - 1);  // wave-uniform
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + (uint32_t)q * 1024u);
      if (i < G::WCH / kRingWaves) {
        // W rows are row-major
        const int row = 16 * q + lrow;
        ring_dma(rw, m0, (row * P.K + k0) * 2 + 16 * ring_piece(row, lpos));
      } else {
        // the hidden copy is k-slice-major ([K/32][Mp][32]); chunks past the
        // row tiles read the last real one
        const int row = 16 * min(q - G::WCH, mtiles - 1) + lrow;
        ring_dma(rh, m0, ((k0 / 32) * P.Mp + row) * 64 + 16 * ring_piece(row, lpos));
      }
    }
  };
  f32x4 acc[NA][NT];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < G::AHEAD; ++s) issue(kb + s);
  for (int s = kb; s < ke; ++s) {
    // this wave's share of stage s has landed; after the barrier everyone's
    // has, and everyone has finished reading stage s - 1, whose slot the
    // loads of stage s + AHEAD then take
    wait_vmcnt<(G::AHEAD - 1) * G::PER>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(s + G::AHEAD);
    const char* stage = ring + (s % G::STAGES) * G::SB;
    u32x4 A[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const int row = 64 * vg + 16 * a + n;
      A[a] = *reinterpret_cast<const u32x4*>(stage + row * 64 + 16 * ring_piece(row, qg));
    }
    // every row tile of the group, real or not: the stage's hidden chunks
    // past the real ones hold copies of the last one, so the products of a
    // padding tile are finite and never stored, and the loop has no branch
    // that would keep the reads of one tile from overlapping the products
    // of another
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = 16 * (mt0 + t) + n;  // hidden row = its row in the hidden part of the stage
      const u32x4 B = *reinterpret_cast<const u32x4*>(stage + G::WCH * 1024 + row * 64 + 16 * ring_piece(row, qg));
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a][t] = mfma_bf16(A[a], B, acc[a][t]);
    }
  }
  wait_vmcnt<0>();  // nothing may land after the ring is reused below (or the workgroup has gone)
  if (part >= 0) {
    // a part of a slice: its products go to the workspace, lane-major, as
    // buffer stores (one lane offset, a scalar offset per tile: per-store
    // 64-bit addresses would take a hundred registers)
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<f32x4*>(P.part) + ((size_t)part * kRingWaves + wave) * NA * NT * 64, (short)0,
        NA * NT * 64 * 16, 0x00020000);
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 v = acc[a][t];
        const u32x4 bits = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(bits, dst, lane * 16, (a * NT + t) * 1024, 0);
      }
    return;
  }
  __syncthreads();
  ring_finish<NT, VG>(P, acc, slice, ring, lane, wave);
}

// K-split slices: one wave per (slice P.full + j, ring wave w) adds the
// P.split parts of that wave's products in part order and takes the best of
// each of its rows, as the ring kernel's epilogue does; its keys go to key
// slot P.full + j * VG + w % VG (rows of its row group only; the VG vocab
// groups of a slice each have a slot, and the reduce kernel takes the best
// over all slots).
template <int NT, int VG>
__global__ __launch_bounds__(64) void vocab_fixup_kernel(const VocabParams P) {
  using G = RingGeo<NT, VG>;
  constexpr int NA = 4;
  const int lane = threadIdx.x, n = lane & 15, qg = lane >> 4;
  const int j = blockIdx.x / kRingWaves, w = blockIdx.x % kRingWaves, vg = w % VG, mg = w / VG;
  const int slice = P.full + j, mt0 = mg * NT, mtiles = P.Mp / 16;
  const size_t pstride = (size_t)kRingWaves * NA * NT * 64;  // f32x4 per part
  const f32x4* src = reinterpret_cast<const f32x4*>(P.part) + (size_t)j * P.split * pstride + (size_t)w * NA * NT * 64 + lane;
  f32x4 acc[NA][NT];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[a][t] = src[(a * NT + t) * 64];
  for (int p = 1; p < P.split; ++p) {
    f32x4 nxt[NA][NT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t) nxt[a][t] = src[p * pstride + (a * NT + t) * 64];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[a][t] = acc[a][t] + nxt[a][t];
  }
  int mrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) mrow[t] = 16 * (mt0 + t);
  uint64_t* keys = P.keys + (size_t)(P.full + j * VG + vg) * P.M;
  epilogue<NA, NT>(P, acc, slice * G::ROWS + 64 * vg, mrow, lane, P.V, [&](int t, uint64_t k) {
    const int m = 16 * (mt0 + t) + n;
    if (qg == 0 && mt0 + t < mtiles && m < P.M) keys[m] = k;
  });
}

// Band kernel, M <= 32 (the draft step): the stream kernel's equal shares of
// the vocabulary's 16-row tiles (one workgroup per CU), but W moves through
// a two-stage LDS ring of 64-wide k slices, 128 bytes of each row: whole
// cache lines, so the loads can be non-temporal (a plain read of W streams
// at 6.1 TB/s with the stream kernel's register layout, 64 bytes of a line
// per instruction and the default policy, against 6.9 TB/s with whole lines
// and non-temporal direct-to-LDS loads). Every wave issues its share of a
// stage's 1 KB loads (8 rows x 128 bytes; lane l fills row l / 8, 16-byte
// unit l % 8 with the row's unit (l % 8) ^ (row % 8), so the 16 rows of an
// operand read hit distinct banks in pairs), waits for them, meets the
// others at the stage barrier and issues the next stage into the other slot
// (which everyone has finished reading). The hidden rows are read from
// global memory per stage (L2 hits), right after the stage's W loads, so
// waiting for them is waiting for the stage; with ROUND (one m-tile, M <= 8)
// they are fp32 rounded in registers, otherwise the bf16 copy.
constexpr int kBandWaves = 8;
constexpr int kBandMaxTiles = 38;  // tiles per share: two stages of 76 KB
constexpr int kBandStage = kBandMaxTiles * 16 * 128;

// One 1 KB non-temporal direct-to-LDS load (see ring_dma).
__device__ __forceinline__ void band_dma(const int (&rsrc)[4], uint32_t m0, int voff) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 r = {rsrc[0], rsrc[1], rsrc[2], rsrc[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(m0), "s"(r)
      : "memory");
}

template <int MS, int NA, bool ROUND>
__global__ __launch_bounds__(64 * kBandWaves, 1) void vocab_band_kernel(const VocabParams P) {
  static_assert(NA * kBandWaves >= kBandMaxTiles, "the waves cover a share");
  static_assert(!ROUND || MS == 1, "rounding in registers with one m-tile");
  __shared__ __attribute__((aligned(1024))) char ring[2 * kBandStage];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const long ntv = (P.V + 15) / 16;
  const int t_lo = (int)(blockIdx.x * ntv / gridDim.x), t_hi = (int)((blockIdx.x + 1) * ntv / gridDim.x);
  const int nch = 2 * (t_hi - t_lo);  // 1 KB chunks per stage (at most 2 kBandMaxTiles, by the plan)
  const int tfirst = t_lo + wave * NA;
  const int vbase = tfirst * 16;
  const int vlim = min(P.V, t_hi * 16);
  const int nk = P.K / 64;
  // W rows [16 t_lo, min(16 t_hi, V)); rows past the vocabulary read as zero
  const uint64_t wb = reinterpret_cast<uint64_t>(P.w) + (uint64_t)t_lo * 16u * (uint64_t)P.K * 2u;
  const int rw[4] = {(int)__builtin_amdgcn_readfirstlane((uint32_t)wb),
                     (int)(__builtin_amdgcn_readfirstlane((uint32_t)(wb >> 32)) & 0xFFFFu),
                     (int)__builtin_amdgcn_readfirstlane((uint32_t)(vlim - t_lo * 16) * (uint32_t)P.K * 2u),
                     0x00020000};
  const uint32_t ring0 = lds_addr(ring);
  const int lrow = lane >> 3, lu = lane & 7;
  // W loads of stage s (k slice s): chunks wave, wave + 8, ... of the
  // share (the stage wait is a full one, so waves may issue different
  // numbers); past the last stage the last slice again into the slot no
  // step reads
  auto issue_w = [&](int s) {
    const uint32_t slot = ring0 + (uint32_t)((s & 1) * kBandStage);
    const int k0 = min(s, nk - 1) * 64;
    for (int c = wave; c < nch; c += kBandWaves) {
      const int row = 8 * c + lrow;
      band_dma(rw, __builtin_amdgcn_readfirstlane(slot + (uint32_t)c * 1024u),
               row * P.K * 2 + k0 * 2 + 16 * (lu ^ (row & 7)));
    }
  };
  // hidden operands of stage s: m-tile t, k-step kk (32 wide) of the slice
  using HRaw = std::conditional_t<ROUND, f32x4[MS][2][2], u32x4[MS][2]>;
  auto load_h = [&](HRaw& H, int s) {
    const int k0 = min(s, nk - 1) * 64;
#pragma unroll
    for (int t = 0; t < MS; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if constexpr (ROUND) {
          const float* hp = P.h + (size_t)min(16 * t + n, P.M - 1) * P.K + k0 + 32 * kk + 8 * qg;
          H[t][kk][0] = *reinterpret_cast<const f32x4*>(hp);
          H[t][kk][1] = *reinterpret_cast<const f32x4*>(hp + 4);
        } else {
          H[t][kk] = *reinterpret_cast<const u32x4*>(P.hb + (size_t)(16 * t + n) * P.K + k0 + 32 * kk + 8 * qg);
        }
      }
  };
  auto to_bf16 = [&](const HRaw& H, u32x4 (&B)[MS][2]) {
#pragma unroll
    for (int t = 0; t < MS; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if constexpr (ROUND) {
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
  f32x4 acc[NA][MS];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < MS; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's tiles in the share (slots past it compute on the last tile
  // and store nothing): LDS rows of tile a
  int arow[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) arow[a] = 16 * (min(tfirst + a, t_hi - 1) - t_lo) + n;
  HRaw H;
  u32x4 B[MS][2];
  issue_w(0);
  load_h(H, 0);
  for (int s = 0; s < nk; ++s) {
    // this wave's loads of stage s have landed (W and hidden); after the
    // barrier everyone's have, and everyone has finished reading stage
    // s - 1, whose slot stage s + 1 then takes
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    to_bf16(H, B);
    issue_w(s + 1);
    load_h(H, s + 1);
    const char* stage = ring + (s & 1) * kBandStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(stage + arow[a] * 128 + 16 * ((4 * kk + qg) ^ (arow[a] & 7)));
#pragma unroll
        for (int t = 0; t < MS; ++t) acc[a][t] = mfma_bf16(A, B[t][kk], acc[a][t]);
      }
  }
  wait_vmcnt<0>();  // nothing may land after the workgroup has gone
  int mrow[MS];
#pragma unroll
  for (int t = 0; t < MS; ++t) mrow[t] = 16 * t;
  uint64_t best[MS];
  epilogue<NA, MS>(P, acc, vbase, mrow, lane, vlim, [&](int t, uint64_t k) { best[t] = k; });
  __syncthreads();  // the ring is free: every wave has left the loop
  uint64_t* red = reinterpret_cast<uint64_t*>(ring);  // [kBandWaves][16 MS]
#pragma unroll
  for (int t = 0; t < MS; ++t)
    if (qg == 0) red[wave * 16 * MS + 16 * t + n] = best[t];
  __syncthreads();
  for (int m = threadIdx.x; m < P.M; m += 64 * kBandWaves) {
    uint64_t k = red[m];
#pragma unroll
    for (int w = 1; w < kBandWaves; ++w) k = red[w * 16 * MS + m] > k ? red[w * 16 * MS + m] : k;
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


}  // namespace

struct VocabPlan {
  bool stream;
  bool band;  // stream: the band kernel (W through LDS in 64-wide k slices) instead
  int ms;     // stream: m-tiles
  int na;     // stream: vocab tiles of 16 rows per wave
  bool round; // stream: hidden rows rounded in registers (one m-tile, M <= 8)
  int tiled;  // tiled: m-tiles per wave (0 = not tiled)
  int ring;   // ring: row tiles per row group (0 = not the ring kernel)
  int rvg;    // ring: vocab groups of 64 rows
  int full;   // ring: slices done whole (the rest in `split` k parts each)
  int split;  // ring: k parts of each slice from `full` on (1: none)
  int nkeys;  // key slots per row: nwg, or full + (nwg - full) * rvg with k parts
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
    // Workgroups take equal shares of the vocabulary tiles (16 rows), as
    // many rounds of the 256 CUs as the largest tile count per wave needs
    // (five with one m-tile, four with two: registers), so every CU streams
    // about the same number of W rows (a vocabulary of 152064 rows: 256
    // workgroups of 37 or 38 tiles instead of 238 of 40 and 18 idle CUs);
    // then the fewest tiles per wave that hold a share.
    const long ntv = (V + 15) / 16;
    const int na_max = mt == 1 ? 5 : 4;
    const long rounds = (ntv + 8L * na_max * kVocabCUs - 1) / (8L * na_max * kVocabCUs);
    const long nwg = std::min(rounds * kVocabCUs, ntv);
    const long share = (ntv + nwg - 1) / nwg;  // tiles of the largest share
    const long need = (share + kStreamWaves - 1) / kStreamWaves;
    p.na = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 5;
    p.nwg = (int)nwg;
    p.round = M <= 8;
    // the band kernel holds a share of at most kBandMaxTiles tiles per
    // stage and keeps one stage in flight, enough for the latency only from
    // about 32 tiles (64 KB) on (measured: a 152064-entry vocabulary, shares
    // of 38 tiles, 268.7 -> 242.6 us; 128256 entries, 32 tiles, 180.1 ->
    // 177.0 us; 32768 entries, 8 tiles, 56.6 -> 79.7 us, so the stream
    // kernel keeps small shares)
    p.band = share >= 32 && share <= kBandMaxTiles && K % 64 == 0;
    // (rounding 16 fp32 hidden rows in the band kernel instead of reading
    // the bf16 copy measured 242 -> 259 us, so it keeps M <= 8 too)
  } else if (kTiledEnabled && mt <= 18) {
    p.stream = false;
    p.tiled = mt <= 6 ? 3 : mt <= 12 ? 6 : 9;
    p.nwg = (V + kTRows - 1) / kTRows;
  } else {
    // the row groups of NT tiles cover every row tile (the padding tiles'
    // products are wasted, so NT is the smallest that covers them): four
    // vocab groups of 64 rows up to 18 and for 21 to 26 row tiles, two vocab groups (a workgroup of 128 vocab rows and
    // four row groups) for 19, 20, 27 and 28 (measured: M = 300 654 us
    // against 765 us with four groups of 13; M = 416 753 us with four groups
    // of 13 against 793 us with two of 7)
    p.stream = false;
    if (mt <= 18) {
      p.ring = mt <= 4 ? 2 : (mt + 1) / 2;
      p.rvg = 4;
    } else if (mt <= 20) {
      p.ring = 5;
      p.rvg = 2;
    } else if (mt <= 26) {
      p.ring = 13;
      p.rvg = 4;
    } else {
      p.ring = 7;
      p.rvg = 2;
    }
    p.nwg = (V + 64 * p.rvg - 1) / (64 * p.rvg);
    // A workgroup fills a CU, so the slices run in rounds of the 256 CUs.
    // When the last round would leave half of them or more idle, each of
    // its slices is cut into split parts of the k range (at least 8 k
    // slices each) that fill the CUs, and a fixup kernel sums the parts
    // (M = 416: 594 slices, the third round's 82 take 246 workgroups).
    const int left = (int)(p.nwg % kVocabCUs), nk = K / 32;
    p.full = p.nwg;
    p.split = 1;
    if (left > 0 && 2 * left <= kVocabCUs) {
      const int sp = std::min((int)(kVocabCUs / left), nk / 8);
      if (sp >= 2) {
        p.full = p.nwg - left;
        p.split = sp;
      }
    }
  }
  p.nkeys = p.ring && p.split > 1 ? p.full + (p.nwg - p.full) * p.rvg : p.nwg;
  return p;
}

// Bytes of the ring kernel's k-split parts (their fp32 products).
static size_t vocab_part_bytes(const VocabPlan& p) {
  if (!p.ring || p.split < 2) return 0;
  return (size_t)(p.nwg - p.full) * p.split * kRingWaves * 4 * p.ring * 64 * sizeof(f32x4);
}

int vocab_max_rows() { return 28 * 16; }

size_t vocab_ws_bytes(int M, int K, int V) {
  const VocabPlan p = vocab_plan(M, K, V);
  return align_up((size_t)p.Mp * K * 2, 256) + align_up((size_t)p.nkeys * M * 8, 256) + align_up(vocab_part_bytes(p), 256);
}

// The ring kernel over whole slices and k parts, then (with parts) the fixup
// kernel; start / stop (may be null) bracket both.
template <int NT, int VG>
static vc_status launch_ring(const VocabPlan& plan, const VocabParams& P, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop) {
  const bool parts = plan.split > 1;
  const dim3 block(64 * kRingWaves);
  const dim3 grid(plan.full + (plan.nwg - plan.full) * plan.split);
  launch_ev(vocab_ring_kernel<NT, VG>, grid, block, 0, stream, start, parts ? nullptr : stop, P);
  if (!parts) return VC_OK;
  const vc_status st = check_launch("vocab projection");
  if (st != VC_OK) return st;
  launch_ev(vocab_fixup_kernel<NT, VG>, dim3((plan.nwg - plan.full) * kRingWaves), dim3(64), 0, stream, nullptr, stop,
            P);
  return check_launch("vocab k-part fixup");
}

vc_status vocab_launch(int M, int K, int V, const float* h, const void* w, int32_t* argmax, float* max_logit,
                       float* logits, void* ws, hipStream_t stream) {
  const VocabPlan plan = vocab_plan(M, K, V);
  VocabParams P{};
  P.h = h;
  P.hb = static_cast<uint16_t*>(ws);
  P.keys = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + align_up((size_t)plan.Mp * K * 2, 256));
  P.part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)plan.Mp * K * 2, 256) +
                                    align_up((size_t)plan.nkeys * M * 8, 256));
  P.full = plan.full;
  P.split = plan.split;
  P.w = static_cast<const uint16_t*>(w);
  P.argmax = argmax;
  P.max_logit = max_logit;
  P.logits = logits;
  P.M = M;
  P.Mp = plan.Mp;
  P.K = K;
  P.V = V;
  P.nwg = plan.nkeys;  // key slots the reduce kernel reads
  P.hb_sliced = plan.ring ? 1 : 0;
  const Timing tm = take_timing();
  const bool main_only = tm.scope == VC_TIME_MAIN_KERNEL;
  vc_status st = VC_OK;
  hipEvent_t mstart = main_only ? tm.start : nullptr, mstop = main_only ? tm.stop : nullptr;
  // the stream kernel may round the hidden rows itself; the others read the
  // bf16 copy
  const bool convert = !plan.stream || !plan.round;
  if (convert) {
    const size_t n = (size_t)plan.Mp * K;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    launch_ev(hidden_to_bf16_kernel, dim3(blocks), dim3(256), 0, stream, main_only ? nullptr : tm.start, nullptr, P);
  }
  if (plan.stream && plan.band) {
    hipEvent_t start = (main_only || convert) ? mstart : tm.start;
    const dim3 grid(plan.nwg), block(64 * kBandWaves);
    if (plan.ms == 1 && plan.round) launch_ev(vocab_band_kernel<1, 5, true>, grid, block, 0, stream, start, mstop, P);
    else if (plan.ms == 1) launch_ev(vocab_band_kernel<1, 5, false>, grid, block, 0, stream, start, mstop, P);
    else launch_ev(vocab_band_kernel<2, 5, false>, grid, block, 0, stream, start, mstop, P);
  } else if (plan.stream) {
    const dim3 block(64 * kStreamWaves);
    hipEvent_t start = (main_only || convert) ? mstart : tm.start;
    const dim3 grid(plan.nwg);
    if (plan.ms == 1 && plan.round) {
      switch (plan.na) {
        case 1: launch_ev(vocab_stream_kernel<1, 1, true>, grid, block, 0, stream, start, mstop, P); break;
        case 2: launch_ev(vocab_stream_kernel<1, 2, true>, grid, block, 0, stream, start, mstop, P); break;
        case 4: launch_ev(vocab_stream_kernel<1, 4, true>, grid, block, 0, stream, start, mstop, P); break;
        default: launch_ev(vocab_stream_kernel<1, 5, true>, grid, block, 0, stream, start, mstop, P); break;
      }
    } else if (plan.ms == 1) {
      switch (plan.na) {
        case 1: launch_ev(vocab_stream_kernel<1, 1, false>, grid, block, 0, stream, start, mstop, P); break;
        case 2: launch_ev(vocab_stream_kernel<1, 2, false>, grid, block, 0, stream, start, mstop, P); break;
        case 4: launch_ev(vocab_stream_kernel<1, 4, false>, grid, block, 0, stream, start, mstop, P); break;
        default: launch_ev(vocab_stream_kernel<1, 5, false>, grid, block, 0, stream, start, mstop, P); break;
      }
    } else {
      switch (plan.na) {
        case 1: launch_ev(vocab_stream_kernel<2, 1, false>, grid, block, 0, stream, start, mstop, P); break;
        case 2: launch_ev(vocab_stream_kernel<2, 2, false>, grid, block, 0, stream, start, mstop, P); break;
        default: launch_ev(vocab_stream_kernel<2, 4, false>, grid, block, 0, stream, start, mstop, P); break;
      }
    }
  } else if (plan.ring) {
    switch (plan.ring * 16 + plan.rvg) {
      case 2 * 16 + 4: st = launch_ring<2, 4>(plan, P, stream, mstart, mstop); break;
      case 3 * 16 + 4: st = launch_ring<3, 4>(plan, P, stream, mstart, mstop); break;
      case 4 * 16 + 4: st = launch_ring<4, 4>(plan, P, stream, mstart, mstop); break;
      case 5 * 16 + 4: st = launch_ring<5, 4>(plan, P, stream, mstart, mstop); break;
      case 6 * 16 + 4: st = launch_ring<6, 4>(plan, P, stream, mstart, mstop); break;
      case 7 * 16 + 4: st = launch_ring<7, 4>(plan, P, stream, mstart, mstop); break;
      case 8 * 16 + 4: st = launch_ring<8, 4>(plan, P, stream, mstart, mstop); break;
      case 9 * 16 + 4: st = launch_ring<9, 4>(plan, P, stream, mstart, mstop); break;
      case 13 * 16 + 4: st = launch_ring<13, 4>(plan, P, stream, mstart, mstop); break;
      case 5 * 16 + 2: st = launch_ring<5, 2>(plan, P, stream, mstart, mstop); break;
      default: st = launch_ring<7, 2>(plan, P, stream, mstart, mstop); break;
    }
    if (st != VC_OK) return st;
  } else {
    const dim3 grid(plan.nwg), block(64 * kTiledWaves);
    if (plan.tiled == 3) launch_ev(vocab_tiled_kernel<3>, grid, block, 0, stream, mstart, mstop, P);
    else if (plan.tiled == 6) launch_ev(vocab_tiled_kernel<6>, grid, block, 0, stream, mstart, mstop, P);
    else launch_ev(vocab_tiled_kernel<9>, grid, block, 0, stream, mstart, mstop, P);
  }
  st = check_launch("vocab projection");
  if (st != VC_OK) return st;
  launch_ev(vocab_reduce_kernel, dim3(M), dim3(256), 0, stream, nullptr, main_only ? nullptr : tm.stop, P);
  return check_launch("vocab argmax reduce");
}

}  // namespace vc
