// Verification attention over the full bf16 cache (VeriCache summary, "Core
// algorithm": one forward pass with KV_full checks all drafted tokens in
// parallel; "P1": verification loads the full cache and is also
// compute-bound, since every cached token meets (k+1)*g query rows).
//
// Work decomposition: one workgroup per (context split, KV head, sequence),
// one per CU (its LDS ring keeps a second one out). All R = n_rows * g query
// rows of the KV head (row = j * g + head, j the draft position) live in the
// workgroup, RT row tiles of 16 per row group, so each K/V tile is read from
// HBM once for every row tile. K/V move in 32-token tiles through an LDS
// ring filled by direct-to-LDS buffer loads issued by two producer waves (K
// and V halves; no registers); only the producers issue such loads, so the
// consumers' LDS reads never wait on them. Up to 9 row tiles, each row group
// has two consumer waves that take the even and odd tiles of each two-tile
// step (8-stage ring): a SIMD then holds waves of two groups, whose softmax
// (VALU) and products (MFMA) overlap; the pair's states merge through LDS at
// the end. Beyond 9 row tiles, one wave per group takes every tile (6-stage
// ring).
//   QK: S^T[token][row] on v_mfma_f32_16x16x32_bf16, A = 16 key rows (LDS,
//       rows XOR-swizzled in 16-byte units so the 16 rows of a read hit
//       distinct banks), B = 16 query rows (registers, exact bf16).
//   softmax: log2 domain; the 1/sqrt(D) * log2(e) scale is folded into the
//       exponent's FMA; the probabilities go to fp16 (11 significant bits;
//       bf16's 8 leave a relative error of about 1e-3 in the output), and
//       the row sums come from one more MFMA of P^T with a ones operand (the
//       same fp16 probabilities as the numerator).
//   PV: O^T[channel][row] += V^T[channel][token] * P^T[token][row] on
//       v_mfma_f32_16x16x32_f16; the V^T operand comes straight from the
//       row-major V tile through the gfx950 transposing LDS read (four token
//       slots of one channel per lane). V tiles go to a ring of their own
//       and are converted to fp16 in place once landed: by the two
//       producers, which load V one step ahead of K so that the conversion
//       has a whole step to finish, or with no producers by the waves that
//       loaded them. The conversion's VALU work is what this costs (measured
//       about 6% of the kernel with producers, 16% without).
// The draft block (x_0..x_k's own keys/values) follows the context tiles of
// the last split of the END call, with the causal mask (row j sees block
// rows 0..j). Per-split partials (max, sum, unnormalised output) are folded
// in split order into a running state kept in the workspace, which allows
// the context to arrive in staged chunks over several calls.
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
  int B, Hq, Hkv, g, NR, R, S, tps, flags;
  float qscale;
};

constexpr int kTT = 32;  // tokens per tile

template <int D>
struct Tile {
  static constexpr int KB = kTT * D * 2;        // bytes of the K (or V) half of a stage
  static constexpr int CHUNKS = KB / 1024;      // 1 KB direct-to-LDS loads per half
  static constexpr int UPR = D / 8;             // 16-byte units per row
  static constexpr int RPC = 1024 / (D * 2);    // rows per 1 KB chunk
};

// LDS unit of (row, 16-byte unit u): XOR swizzle within the row.
template <int D>
__device__ __forceinline__ int swz(int row, int u) {
  return u ^ (row & (Tile<D>::UPR - 1));
}

// s_waitcnt on the vector-memory counter only: vmcnt(N), others untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// One segment of tiles: K and V rows at a fixed byte stride, rows past the
// segment's extent read as zero (buffer range check).
struct Segment {
  const uint16_t *k, *v;
  uint32_t bytes;  // extent of each of k and v
  int row_bytes;
  int ntiles;
};

__device__ __forceinline__ uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Issue the direct-to-LDS load of 1 KB chunk c of the K (half 0) or V
// (half 1) part of one tile into that half's ring slot dst. Lane l of chunk c fills LDS unit 64c + l, i.e.
// row RPC*c + l / UPR, unit l % UPR, with the global unit that the swizzle
// puts there. Every operand that is wave-uniform is made visibly so (the
// buffer resource must sit in scalar registers).
template <int D>
__device__ __forceinline__ void issue_chunk(char* dst, const Segment& sg, int tile, int lane, int half, int c) {
  using T = Tile<D>;
  const uint64_t a = reinterpret_cast<uint64_t>(half ? sg.v : sg.k);
  const uint64_t au = ((uint64_t)uni((uint32_t)(a >> 32)) << 32) | uni((uint32_t)a);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(au), (short)0, (int)uni(sg.bytes), 0x00020000);
  const int rb = (int)uni((uint32_t)sg.row_bytes), t0 = (int)uni((uint32_t)(tile * kTT));
  const int rl = lane / T::UPR, ul = lane % T::UPR;
  const int row = T::RPC * c + rl;
  const int voff = (t0 + row) * rb + swz<D>(row, ul) * 16;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + c * 1024), 16, voff, 0, 0, kStreamPolicy);
}

// The same load for a wave that also reads the ring (consumer-issued
// loads): written as an asm statement, so the compiler does not count it as
// a pending write to LDS and does not wait for it (vmcnt(0)) before this
// wave's reads of other stages. The asm has no register outputs; the caller
// orders the data with explicit vmcnt waits and a barrier. M0 takes the
// stage address (one wait state before the load reads it) and is restored.
template <int D>
__device__ __forceinline__ void issue_chunk_asm(char* dst, const Segment& sg, int tile, int lane, int half,
                                                int c) {
  using T = Tile<D>;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t a = reinterpret_cast<uint64_t>(half ? sg.v : sg.k);
  // buffer descriptor: base, stride 0, extent in bytes, the same flags as
  // the descriptors built for issue_chunk
  const i32x4 rsrc = {(int)uni((uint32_t)a), (int)(uni((uint32_t)(a >> 32)) & 0xFFFFu), (int)uni(sg.bytes),
                      0x00020000};
  const int rb = (int)uni((uint32_t)sg.row_bytes), t0 = (int)uni((uint32_t)(tile * kTT));
  const int rl = lane / T::UPR, ul = lane % T::UPR;
  const int row = T::RPC * c + rl;
  const int voff = (t0 + row) * rb + swz<D>(row, ul) * 16;
  const uint32_t m0 = uni(lds_addr(dst + c * 1024));
  // M0 is reserved to the compiler (a clobber of it is not honoured), so the
  // statement puts its value back after the load has read it
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(m0), "s"(rsrc)
      : "memory");
}

// A whole half of a tile: one producer wave per half. The producers also
// convert landed V tiles in LDS while later loads are in flight, so they
// issue the asm form (no wait for pending loads before their LDS accesses).
template <int D>
__device__ __forceinline__ void issue_half(char* dst, const Segment& sg, int tile, int lane, int half) {
#pragma unroll
  for (int c = 0; c < Tile<D>::CHUNKS; ++c) issue_chunk_asm<D>(dst, sg, tile, lane, half, c);
}

// One landed 1 KB chunk of V rows to fp16 in place (16 bytes per lane). A
// bf16 value converts exactly when 2^-17 <= |v| <= 65504; smaller ones
// round to fp16's 2^-24 grid, larger ones become infinite.
__device__ __forceinline__ void chunk_to_f16(char* chunk, int lane) {
  u32x4* p = reinterpret_cast<u32x4*>(chunk + lane * 16);
  const u32x4 w = *p;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_f16(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xFFFF0000u));
  *p = o;
}

// lgkmcnt(0): this wave's LDS accesses have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Raw scores s (unscaled q.k, -inf where masked) of one tile become
// p = 2^(s * qscale - m + kProbShift). The running max moves only when the
// tile's max exceeds it by more than kRescaleThreshold, which keeps the
// accumulator rescale rare; the result is the same softmax. The shift puts
// the largest p (2^15) just inside fp16's range, so the fp16 probabilities
// lose only terms below 2^-24, i.e. 2^-31 of the running max or less, and
// keep 11 significant bits down to 2^-14 (2^-21 of the max). Numerator and
// row sums carry the same factor 2^kProbShift, on every split alike.
constexpr float kProbShift = 7.0f;
static_assert(kRescaleThreshold + kProbShift <= 15.0f, "largest probability inside fp16's range");

// Online-softmax state of RT row tiles. The row sums live in an MFMA
// accumulator (lsum): P^T contracted with a ones operand, so each sum is
// complete after the MFMA (no cross-lane reduction) and uses the same fp16
// probabilities as the numerator.
template <int RT, int MT>
struct VState {
  float m[RT];   // running max (log2 domain, scaled), identical on all lanes of a column
  float nm[RT];  // exponent offset kProbShift - m (kProbShift while m is -inf)
  float th[RT];  // rescale threshold in raw score units: (m + kRescaleThreshold) / qscale
  f32x4 acc[RT][MT];
  f32x4 lsum[RT];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m[rt] = kNegInf;
      nm[rt] = kProbShift;
      th[rt] = kNegInf;
      lsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Maximum that propagates NaN (v_maximum3_f32): unlike fmaxf it needs no
// canonicalising of operands that come from the MFMA or a lane permute.
// Scores are finite or -inf on every row whose result is kept.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax_q(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The tile's raw maxima are compared with the threshold kept in raw score
// units, and the exponent offset is kept beside the max, so a tile that
// moves no max costs no scaling of the maxima and no test of an unset max.
template <int RT, int MT>
__device__ __forceinline__ void verify_softmax(VState<RT, MT>& st, float (&s)[RT][2][4], float qscale,
                                               float rqscale) {
  float x[RT];
  bool need = false;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    x[rt] = vmax_q(vmax(vmax(vmax(s[rt][0][0], s[rt][0][1]), vmax(s[rt][0][2], s[rt][0][3])),
                        vmax(vmax(s[rt][1][0], s[rt][1][1]), vmax(s[rt][1][2], s[rt][1][3]))));
    need = need || (x[rt] > st.th[rt]);
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bool up = x[rt] > st.th[rt];
      const float bm = x[rt] * qscale;
      const float alpha = up ? fast_exp2(st.m[rt] - bm) : 1.f;
      st.m[rt] = up ? bm : st.m[rt];
      st.nm[rt] = up ? kProbShift - bm : st.nm[rt];
      st.th[rt] = up ? (bm + kRescaleThreshold) * rqscale : st.th[rt];
      st.lsum[rt] *= alpha;
#pragma unroll
      for (int t = 0; t < MT; ++t) st.acc[rt][t] *= alpha;
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // a row that has seen no visible token yet (max still -inf, offset
    // kProbShift) gets p = 0 from its -inf scores
    const float nm = st.nm[rt];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[rt][i][r] = fast_exp2(fmaf(s[rt][i][r], qscale, nm));
  }
}

// One 32-token tile for this wave's RT row tiles (K and V rows at kstage and
// vstage; between() runs once the products are issued). nvalid masks tokens for
// all rows; token t is visible to row tile rt's rows only when t <= lim[rt]
// (the causal limit in the draft block, relative to the tile's first token;
// large for context tiles).
template <int D, int RT, bool MASK, typename Between>
__device__ __forceinline__ void tile_compute(const char* kstage, const char* vstage, int nvalid, int lane,
                                             const uint32_t (&Bq)[RT][D / 32][4], const int (&lim)[RT],
                                             float qscale, float rqscale, VState<RT, D / 16>& st,
                                             Between&& between) {
  constexpr int NG = D / 32, MT = D / 16;
  const int n = lane & 15, qg = lane >> 4;
  float s[RT][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * i + n;
    const char* kr = kstage + row * (D * 2);
    u32x4 A[NG];
#pragma unroll
    for (int kk = 0; kk < NG; ++kk)
      A[kk] = *reinterpret_cast<const u32x4*>(kr + swz<D>(row, qg * NG + kk) * 16);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk)
        c = mfma_bf16(A[kk], u32x4{Bq[rt][kk][0], Bq[rt][kk][1], Bq[rt][kk][2], Bq[rt][kk][3]}, c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * i + 4 * qg + r;
        if constexpr (MASK) s[rt][i][r] = (t < nvalid && t <= lim[rt]) ? c[r] : kNegInf;
        else s[rt][i][r] = c[r];
      }
    }
  }
  verify_softmax<RT, MT>(st, s, qscale, rqscale);
  uint32_t Bp[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r >> 1, rr = 2 * (r & 1);
      Bp[rt][r] = pack_f16(s[rt][i][rr], s[rt][i][rr + 1]);  // p <= 2^15
    }
  // V^T operand: lane n of slot group qg reads token 16h + 4qg + (n >> 2),
  // channels 16m + 4(n & 3) .. + 3; the transposing read hands lane n the
  // four token slots of channel 16m + n (V rows already in fp16).
  const char* vbase = vstage;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t A[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + 4 * qg + (n >> 2);
      const int u = 2 * m + ((n & 3) >> 1);
      const char* p = vbase + row * (D * 2) + swz<D>(row, u) * 16 + (n & 1) * 8;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
      A[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
      A[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      st.acc[rt][m] =
          mfma_f16(u32x4{A[0], A[1], A[2], A[3]}, u32x4{Bp[rt][0], Bp[rt][1], Bp[rt][2], Bp[rt][3]}, st.acc[rt][m]);
    }
  }
  constexpr uint32_t kOnes = 0x3C003C00u;  // two fp16 1.0
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    st.lsum[rt] = mfma_f16(u32x4{kOnes, kOnes, kOnes, kOnes}, u32x4{Bp[rt][0], Bp[rt][1], Bp[rt][2], Bp[rt][3]},
                           st.lsum[rt]);
  between();  // work that can overlap the products still in flight
}

// Consumer waves compute, the last two waves load. Without PAIR, consumer
// wave w holds row tiles RT*w .. RT*w+RT-1 and computes every tile, one tile
// per workgroup barrier. With PAIR, waves w and w + NW (NW row groups) hold
// the same row tiles and take the even and odd tiles of each two-tile step:
// the two waves of a pair sit on different SIMDs next to a wave of another
// pair, so one wave's softmax (VALU) runs while another's products (MFMA)
// do, and the pair's two partial states are merged through LDS at the end.
//
// With SELF (wave pairs, eight consumer waves, no producers) every consumer
// wave issues a fixed share of each step's loads itself, AHEAD steps ahead,
// and waits for its share of the current step before the step's barrier: the
// two producer slots go to a fourth pair of row groups.
//
// V tiles travel one step ahead of the K tiles (AHEAD + 1 steps in flight),
// in a ring one step deeper than the K ring: a slot that a step's V loads
// overwrite held V that was read two steps earlier. The V producer waits
// for the V of step st + 1 before the barrier of step st; between the
// barriers of steps st - 1 and st both producers convert half of step st's
// V chunks each to fp16 (an opening barrier covers step 0). With SELF, each
// wave converts the V chunks of step sp + 1 that it loaded right after the
// barrier of step sp.
template <int D, int RT, bool PAIR, bool SELF>
__global__ __launch_bounds__(512, 2) void verify_kernel(const VerifyParams P) {
  static_assert(!SELF || PAIR, "consumer-issued loads come with wave pairs");
  constexpr int NG = D / 32, MT = D / 16;
  constexpr int TPS = PAIR ? 2 : 1;          // tiles per barrier step
  constexpr int STAGES = PAIR ? 8 : 6;       // K ring depth in tiles
  constexpr int VSTAGES = STAGES + TPS;      // V ring depth in tiles
  constexpr int AHEAD = STAGES / TPS - 2;    // K steps in flight ahead of the one computed
  using T = Tile<D>;
  constexpr int SELF_WAVES = 8;
  constexpr int PER = TPS * 2 * T::CHUNKS / SELF_WAVES;  // 1 KB loads per consumer per step (SELF)
  static_assert(!SELF || PER * SELF_WAVES == TPS * 2 * T::CHUNKS, "even share of a step's loads");
  __shared__ __attribute__((aligned(16))) char ring[(STAGES + VSTAGES) * T::KB];
  auto kslot = [&](int t) { return ring + (t % STAGES) * T::KB; };
  auto vslot = [&](int t) { return ring + (STAGES + t % VSTAGES) * T::KB; };
  const int lane = threadIdx.x & 63, hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ncons = SELF ? SELF_WAVES : blockDim.x / 64 - 2;
  // Roles. With eight waves the producers take waves 0 and 4, which share a
  // SIMD when waves go round-robin to the four SIMDs: the other three SIMDs
  // then hold two consumers each (the most any SIMD holds anyway) and the
  // producers' V conversion runs beside no consumer; waves 1, 2, 3 are
  // consumers 0, 1, 2 and waves 5, 6, 7 consumers 4, 5, 3, so the two waves
  // of a SIMD belong to different row groups. Otherwise the producers are
  // the last two waves. wave: the consumer index 0 .. ncons - 1.
  const bool eight = !SELF && ncons == 6;
  const bool producer = eight ? (hw & 3) == 0 : (!SELF && hw >= ncons);
  const int wave = !eight ? hw : hw < 4 ? hw - 1 : 3 + (hw - 4) % 3;
  const int nw = ncons / TPS;  // row groups
  const int grp = wave % nw, parity = wave / nw;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const size_t unit = (size_t)b * P.Hkv + hk;
  const int n = lane & 15, qg = lane >> 4;

  // segment 0: context rows [r0, r0 + nval) of the chunk, visible below ctx_len
  const int ctx = P.ctx_len[b];
  const int r0 = split * P.tps;
  const int nval = max(0, min(min(r0 + P.tps, P.tok_count), ctx - P.tok_begin) - r0);
  Segment s0;
  s0.k = P.ck + (unit * P.t_cap + min(r0, P.t_cap)) * D;
  s0.v = P.cv + (unit * P.t_cap + min(r0, P.t_cap)) * D;
  s0.bytes = (uint32_t)nval * D * 2;
  s0.row_bytes = D * 2;
  s0.ntiles = (nval + kTT - 1) / kTT;
  // segment 1: the draft block (last split of the END call), causal
  const bool with_block = (P.flags & VC_VERIFY_END) && split == P.S - 1;
  Segment s1;
  const int stride = P.B * P.Hkv * D;
  s1.k = P.k_new + unit * D;
  s1.v = P.v_new + unit * D;
  s1.bytes = (uint32_t)((size_t)P.NR * stride * 2);
  s1.row_bytes = stride * 2;
  s1.ntiles = with_block ? (P.NR + kTT - 1) / kTT : 0;
  const int ntiles = s0.ntiles + s1.ntiles;
  const int nsteps = (ntiles + TPS - 1) / TPS;

  // SELF: this wave's share of one step's loads: waves 4 ti .. 4 ti + 3
  // load tile ti of the step, wave w the same PER / 2 consecutive chunks of
  // its K rows and of its V rows, so every wave converts as many V chunks.
  // A call for step s issues the K chunks of step s and the V chunks of step
  // s + 1 (with V_ONLY, the V chunks of step s alone); past the last tile the
  // last one is loaded again into a slot no step reads
  static_assert(!SELF || (TPS == 2 && PER % 2 == 0 && (PER / 2) * 4 == T::CHUNKS), "SELF chunk shares");
  auto share_chunk = [&](int i, int& ti, int& half, int& c) {
    ti = wave >> 2;
    half = i / (PER / 2);
    c = (wave & 3) * (PER / 2) + i % (PER / 2);
  };
  auto issue_share = [&](int step, bool v_only) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int ti, half, c;
      share_chunk(i, ti, half, c);
      if (v_only && half == 0) continue;
      int t = (step + (half && !v_only ? 1 : 0)) * TPS + ti;
      char* dst = half ? vslot(t) : kslot(t);
      t = min(t, ntiles - 1);
      if (t < s0.ntiles) issue_chunk_asm<D>(dst, s0, t, lane, half, c);
      else issue_chunk_asm<D>(dst, s1, t - s0.ntiles, lane, half, c);
    }
  };
  // SELF: this wave's V chunks of a landed step to fp16
  auto convert_share = [&](int step) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int ti, half, c;
      share_chunk(i, ti, half, c);
      const int t = step * TPS + ti;
      if (half == 1 && t < ntiles) chunk_to_f16(vslot(t) + c * 1024, lane);
    }
  };

  if (producer) {
    // producer: K (first) or V (second) halves, AHEAD (K) or AHEAD + 1 (V)
    // steps ahead
    const int half = eight ? hw >> 2 : hw - ncons;
    auto issue = [&](int t) {
      char* dst = half ? vslot(t) : kslot(t);
      t = min(t, ntiles - 1);  // past the end: reload the last tile into an unused slot
      if (t < s0.ntiles) issue_half<D>(dst, s0, t, lane, half);
      else issue_half<D>(dst, s1, t - s0.ntiles, lane, half);
    };
    if (ntiles > 0) {
      // K: steps 0 .. AHEAD - 1; V: steps 0 .. AHEAD, and V of step 0 landed
      // before an opening barrier
      for (int t = 0; t < (AHEAD + half) * TPS; ++t) issue(t);
      if (half == 1) wait_vm<AHEAD * TPS * T::CHUNKS>();
      __builtin_amdgcn_s_barrier();
      for (int st = 0; st < nsteps; ++st) {
#pragma unroll
        for (int i = 0; i < TPS; ++i) issue((st + AHEAD + half) * TPS + i);
        // this producer's half of the chunks of step st's V tiles to fp16
        // (they landed before the previous barrier)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
          const int t = st * TPS + i;
          if (t < ntiles) {
#pragma unroll
            for (int c = half * (T::CHUNKS / 2); c < (half + 1) * (T::CHUNKS / 2); ++c)
              chunk_to_f16(vslot(t) + c * 1024, lane);
          }
        }
        // K of step st, or V of step st + 1, landed
        wait_vm<AHEAD * TPS * T::CHUNKS>();
        wait_lds();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
      }
      wait_vm<0>();  // nothing may land after the workgroup has gone
    }
    if constexpr (PAIR) {
      // the consumers' two hand-over barriers (the first one also tells them
      // that no load into the ring is in flight any more)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  // query operands of this wave's row tiles (unscaled bf16, exact)
  uint32_t Bq[RT][NG][4];
  int rowj[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * (grp * RT + rt) + n;
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

  // consumers before producers at the instruction arbiter: the producers'
  // V conversion has a whole step to finish and fills the issue gaps
  if constexpr (!SELF) __builtin_amdgcn_s_setprio(1);
  VState<RT, MT> st;
  st.init();
  const float rqscale = 1.f / P.qscale;
  if constexpr (SELF) {
    // the query has landed before the ring starts, so the compiler (which
    // does not see the ring's asm loads) has nothing left to wait for in the
    // loop
    wait_vm<0>();
    if (ntiles > 0) {
      issue_share(0, true);
      for (int sp = 0; sp < AHEAD; ++sp) issue_share(sp, false);
      wait_vm<AHEAD * PER>();  // the V chunks of step 0
      asm volatile("" ::: "memory");
      convert_share(0);
    }
  }
  // One step's barrier. SELF: issue step sp + AHEAD, wait until this wave's
  // share of step sp has landed, then a bare barrier (a workgroup fence would
  // also wait for this wave's loads of the later steps; the asm statements
  // keep the step's LDS reads below the barrier). Otherwise it pairs with the
  // producers' bare barrier; the fence keeps this step's LDS reads below it
  // (consumers have no loads in flight, so it costs nothing).
  // In step sp, SELF converts its V chunks of step sp + 1 (landed with the K
  // chunks of step sp) while the step's products run; those LDS accesses end
  // before the next barrier.
  auto step_sync = [&](int sp) {
    if constexpr (SELF) {
      issue_share(sp + AHEAD, false);
      wait_vm<AHEAD * PER>();
      wait_lds();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };
  auto convert_next = [&](int sp) {
    if constexpr (SELF) convert_share(sp + 1);
  };
  if constexpr (!SELF)
    if (ntiles > 0) __syncthreads();  // the producers' opening barrier
  // steps made of full context tiles need no mask; the partial last context
  // tile and the causal draft-block tiles follow in a second loop
  const int nfull_steps = (nval / kTT) / TPS;
  int lim_all[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) lim_all[rt] = kTT;
  for (int sp = 0; sp < nfull_steps; ++sp) {
    step_sync(sp);
    const int t = sp * TPS + parity;
    tile_compute<D, RT, false>(kslot(t), vslot(t), kTT, lane, Bq, lim_all, P.qscale, rqscale, st,
                               [&] { convert_next(sp); });
  }
  for (int sp = nfull_steps; sp < nsteps; ++sp) {
    step_sync(sp);
    const int t = sp * TPS + parity;
    if (t < ntiles) {
      const bool blk = t >= s0.ntiles;
      const int tb = t - s0.ntiles;
      int lim[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) lim[rt] = blk ? rowj[rt] - tb * kTT : kTT;
      const int nv = blk ? min(kTT, P.NR - tb * kTT) : min(kTT, nval - t * kTT);
      tile_compute<D, RT, true>(kslot(t), vslot(t), nv, lane, Bq, lim, P.qscale, rqscale, st,
                                [&] { convert_next(sp); });
    } else {
      convert_next(sp);
    }
  }

  if constexpr (PAIR) {
    // hand the odd wave's state to the even wave through the (now idle) ring:
    // per row tile MT*4 accumulator words, the max and the sum, lane-major
    // (SELF: every wave's ring loads have landed before the barrier)
    if constexpr (SELF) wait_vm<0>();
    __syncthreads();
    constexpr int WORDS = MT * 4 + 2;
    float* xa = reinterpret_cast<float*>(ring) + (size_t)grp * RT * WORDS * 64 + lane;
    if (parity == 1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) xa[(rt * WORDS + 4 * m + r) * 64] = st.acc[rt][m][r];
        xa[(rt * WORDS + MT * 4) * 64] = st.m[rt];
        xa[(rt * WORDS + MT * 4 + 1) * 64] = st.lsum[rt][0];
      }
    }
    __syncthreads();
    if (parity == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mb = xa[(rt * WORDS + MT * 4) * 64], lb = xa[(rt * WORDS + MT * 4 + 1) * 64];
      const float ma = st.m[rt], mx = vmax(ma, mb);
      const float fa = ma == kNegInf ? 0.f : fast_exp2(ma - mx);
      const float fb = mb == kNegInf ? 0.f : fast_exp2(mb - mx);
      st.m[rt] = mx;
      st.lsum[rt][0] = st.lsum[rt][0] * fa + lb * fb;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[rt][m][r] = st.acc[rt][m][r] * fa + xa[(rt * WORDS + 4 * m + r) * 64] * fb;
    }
  }

  // partial for this split: rows of this wave's row tiles
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * (grp * RT + rt) + n;
    const float l = st.lsum[rt][0];
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

// Fold this call's splits (in order, kBatch at a time: the loads of a batch
// are issued together, every one from a valid split, duplicates masked after
// the load) into the running state; on END write out. A thread takes four
// channels of one row (16-byte loads and stores), a workgroup
// kMergeThreads / (D / 4) rows.
constexpr int kMergeThreads = 256;

template <int D, int kBatch>
__global__ __launch_bounds__(kMergeThreads) void verify_merge_kernel(const VerifyParams P) {
  constexpr int C4 = D / 4, RPW = kMergeThreads / C4;
  const int c = 4 * (threadIdx.x % C4), row = blockIdx.x * RPW + threadIdx.x / C4, hk = blockIdx.y, b = blockIdx.z;
  if (row >= P.R) return;
  const size_t unit = (size_t)b * P.Hkv + hk;
  const size_t rr = unit * P.R + row;
  float M = kNegInf, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  if (!(P.flags & VC_VERIFY_BEGIN)) {
    M = P.run_ml[rr * 2];
    L = P.run_ml[rr * 2 + 1];
    O = *reinterpret_cast<const f32x4*>(P.run_o + rr * D + c);
  }
  for (int s0 = 0; s0 < P.S; s0 += kBatch) {
    float ms[kBatch], ls[kBatch];
    f32x4 os[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const size_t pr = (unit * P.S + min(s0 + i, P.S - 1)) * P.R + row;
      ms[i] = P.part_ml[pr * 2];
      ls[i] = P.part_ml[pr * 2 + 1];
      os[i] = *reinterpret_cast<const f32x4*>(P.part_o + pr * D + c);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) ms[i] = s0 + i < P.S ? ms[i] : kNegInf;
    float mx = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) mx = fmaxf(mx, ms[i]);
    if (mx == kNegInf) continue;  // nothing visible so far
    const float a = M == kNegInf ? 0.f : fast_exp2(M - mx);
    L *= a;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[e] *= a;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const bool ok = ms[i] != kNegInf;
      const float w = ok ? fast_exp2(ms[i] - mx) : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = ok ? fmaf(os[i][e], w, O[e]) : O[e];
      L = ok ? fmaf(ls[i], w, L) : L;
    }
    M = mx;
  }
  if (P.flags & VC_VERIFY_END) {
    const int j = row / P.g, hl = row % P.g;
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (L > 0.f) ? O[e] / L : 0.f;
    *reinterpret_cast<f32x4*>(P.out + (((size_t)j * P.B + b) * P.Hq + (size_t)hk * P.g + hl) * D + c) = r;
  } else {
    *reinterpret_cast<f32x4*>(P.run_o + rr * D + c) = O;
    if (c == 0) {
      P.run_ml[rr * 2] = M;
      P.run_ml[rr * 2 + 1] = L;
    }
  }
}

template <int D>
void launch_verify(const VerifyParams& P, int rt, bool pair, bool self, int nwaves, dim3 grid, hipStream_t s,
                   hipEvent_t start, hipEvent_t stop) {
  const dim3 block(64 * (nwaves + (self ? 0 : 2)));
  if (self) {
    launch_ev(verify_kernel<D, 3, true, true>, grid, block, 0, s, start, stop, P);
  } else if (pair) {
    if (rt == 2) launch_ev(verify_kernel<D, 2, true, false>, grid, block, 0, s, start, stop, P);
    else launch_ev(verify_kernel<D, 3, true, false>, grid, block, 0, s, start, stop, P);
  } else {
    if (rt == 2) launch_ev(verify_kernel<D, 2, false, false>, grid, block, 0, s, start, stop, P);
    else launch_ev(verify_kernel<D, 3, false, false>, grid, block, 0, s, start, stop, P);
  }
}

}  // namespace

struct VerifyPlan {
  int rt, nwaves, tps, s_ctx;
  bool pair, self;
};

// Row tiling: wave pairs with two row tiles per wave up to 6 tiles and three
// up to 9 (plus 2 producers); 10 to 12 tiles, four pairs of three that issue
// their own loads; beyond, one wave per group of three row tiles (at most 6
// consumer waves plus the 2 producers). Every case is 2 waves per SIMD at
// most, with the whole register file for the row tiles' accumulators. Two
// tiles per wave without pairs (more consumer waves) measured slower: every
// consumer reads each whole K/V tile from LDS; so was nine tiles on four
// self-issuing pairs (three empty row tiles: 186 -> 216 us on the Llama-3-8B
// layer). Context split of a call:
// about 256 workgroups (one per CU), whole 32-token tiles, at least 8 tiles
// per split; the draft block rides on the last split. The split count never
// decreases with chunk_tokens, so a workspace sized for the largest chunk
// fits every smaller one.
VerifyPlan verify_plan(const vc_attn_shape& sh, int n_rows, int chunk_tokens) {
  const int R = n_rows * (sh.n_q_heads / sh.n_kv_heads);
  const int tiles = (R + 15) / 16;
  // up to 9 row tiles: wave pairs (at most 3 groups, 6 consumer waves, 2
  // producers); 10 to 12: wave pairs of 4 groups that issue their own loads
  // (8 consumer waves); beyond: one wave per group of three row tiles (at
  // most 6 waves)
  const bool self = tiles >= 10 && tiles <= 12;
  const bool pair = tiles <= 9 || self;
  const int rt = (pair && tiles <= 6) ? 2 : 3;
  const int nwaves = self ? 8 : ((tiles + rt - 1) / rt) * (pair ? 2 : 1);
  const long long units = (long long)sh.batch * sh.n_kv_heads;
  const long long ctx_tiles = ((long long)chunk_tokens + kTT - 1) / kTT;
  long long s_ctx = (256 + units - 1) / units;
  const long long max_s = (ctx_tiles + 7) / 8;
  if (s_ctx > max_s) s_ctx = max_s;
  if (s_ctx < 1) s_ctx = 1;
  const long long tps = ((ctx_tiles + s_ctx - 1) / s_ctx) * kTT;
  return VerifyPlan{rt, nwaves, (int)(tps > 0 ? tps : kTT), (int)s_ctx, pair, self};
}

int verify_max_rows() { return 6 * 3 * 16; }

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
  return run_bytes(sh, R) + part_bytes(sh, R, (size_t)p.s_ctx);
}

vc_status verify_launch(const vc_attn_shape& sh, int n_rows, const void* q, const void* k_new, const void* v_new,
                        const vc_kv_chunk& ctx, const int32_t* ctx_len, int flags, float* out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  const VerifyPlan plan = verify_plan(sh, n_rows, ctx.tok_count);
  VerifyParams P{};
  const size_t R = (size_t)n_rows * (sh.n_q_heads / sh.n_kv_heads);
  const size_t units = (size_t)sh.batch * sh.n_kv_heads;
  const size_t S = (size_t)plan.s_ctx;
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
  P.S = (int)S;
  P.flags = flags;
  P.qscale = kLog2e / sqrtf((float)sh.head_dim);
  const dim3 grid(P.S, sh.n_kv_heads, sh.batch);
  const Timing tm = take_timing();
  const bool main_only = tm.scope == VC_TIME_MAIN_KERNEL;
  if (sh.head_dim == 128)
    launch_verify<128>(P, plan.rt, plan.pair, plan.self, plan.nwaves, grid, stream, tm.start, main_only ? tm.stop : nullptr);
  else
    launch_verify<64>(P, plan.rt, plan.pair, plan.self, plan.nwaves, grid, stream, tm.start, main_only ? tm.stop : nullptr);
  vc_status st = check_launch("verify attention");
  if (st != VC_OK) return st;
  hipEvent_t mstop = main_only ? nullptr : tm.stop;
  const dim3 mblock(kMergeThreads);
  // batches of four when the splits fit one (no duplicate loads), else eight
  if (sh.head_dim == 128) {
    const dim3 mgrid((unsigned)((R + kMergeThreads / 32 - 1) / (kMergeThreads / 32)), sh.n_kv_heads, sh.batch);
    if (P.S <= 4) launch_ev(verify_merge_kernel<128, 4>, mgrid, mblock, 0, stream, nullptr, mstop, P);
    else launch_ev(verify_merge_kernel<128, 8>, mgrid, mblock, 0, stream, nullptr, mstop, P);
  } else {
    const dim3 mgrid((unsigned)((R + kMergeThreads / 16 - 1) / (kMergeThreads / 16)), sh.n_kv_heads, sh.batch);
    if (P.S <= 4) launch_ev(verify_merge_kernel<64, 4>, mgrid, mblock, 0, stream, nullptr, mstop, P);
    else launch_ev(verify_merge_kernel<64, 8>, mgrid, mblock, 0, stream, nullptr, mstop, P);
  }
  return check_launch("verify merge");
}

}  // namespace vc
