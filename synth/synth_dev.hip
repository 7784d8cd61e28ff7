// Device copy of the seeded input generator in synth/__init__.py (SplitMix64
// of Steele, Lea and Flood, OOPSLA 2014, used as a counter-based generator).
// It draws inputs only: context keys/values, the synthetic embedding of a
// token, the vocabulary matrix and token scores. The test suite checks every
// function here bit for bit against the numpy version.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kRoleCtxK = 1, kRoleCtxV = 2, kRoleEmbQ = 3, kRoleEmbK = 4, kRoleEmbV = 5, kRoleW = 6,
                   kRoleScore = 7;
constexpr uint32_t kZScaleBits = 0x37ddb3d6u;  // fp32 nearest to 1/37837.23
constexpr uint32_t kWScaleBits = 0x3ca3d70au;  // fp32 nearest to 0.02

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__device__ __forceinline__ float z_fp32(uint64_t u) {
  const uint32_t s = (uint32_t)(u & 0xFFFF) + (uint32_t)((u >> 16) & 0xFFFF) + (uint32_t)((u >> 32) & 0xFFFF) +
                     (uint32_t)(u >> 48);
  const float c = (float)((int)s - 131070);
  return __fmul_rn(c, __uint_as_float(kZScaleBits));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t role, uint64_t idx) {
  return splitmix64(key + ((role << 56) | idx));
}

__device__ __forceinline__ uint16_t to_out(float x, int fp16) {
  if (fp16) return __builtin_bit_cast(uint16_t, (_Float16)x);
  return bf16_rne(x);
}

// Context K or V: out bf16 [B][Hkv][t_cap][D], rows [0, T) filled.
__global__ void fill_ctx_kernel(uint64_t seed, uint64_t role, int B, int Hkv, int T, int D, int t_cap,
                                const float* key_mult, uint16_t* out) {
  const uint64_t key = splitmix64(seed);
  const size_t total = (size_t)B * Hkv * T * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(i % D);
    const size_t r = i / D;
    const int t = (int)(r % T);
    const size_t u = r / T;
    const int h = (int)(u % Hkv), b = (int)(u / Hkv);
    const uint64_t idx = ((((uint64_t)b << 8) | (uint64_t)h) << 40) | ((uint64_t)t << 16) | (uint64_t)d;
    uint16_t v = bf16_rne(z_fp32(draw(key, role, idx)));
    if (key_mult != nullptr) v = bf16_rne(__uint_as_float((uint32_t)v << 16) * key_mult[h * D + d]);
    out[(u * t_cap + t) * D + d] = v;
  }
}

__global__ void fill_w_kernel(uint64_t seed, int V, int H, uint16_t* out) {
  const uint64_t key = splitmix64(seed);
  const size_t total = (size_t)V * H;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const uint64_t n = i / H, k = i % H;
    const float z = z_fp32(draw(key, kRoleW, (n << 32) | k));
    out[i] = bf16_rne(__fmul_rn(z, __uint_as_float(kWScaleBits)));
  }
}

__global__ void fill_scores_kernel(uint64_t seed, int B, int Hkv, int T, float* out) {
  const uint64_t key = splitmix64(seed);
  const size_t total = (size_t)B * Hkv * T;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i % T);
    const size_t u = i / T;
    const int h = (int)(u % Hkv), b = (int)(u / Hkv);
    const uint64_t idx = ((((uint64_t)b << 8) | (uint64_t)h) << 24) | (uint64_t)t;
    const uint64_t r = draw(key, kRoleScore, idx);
    const double uu = (double)((r >> 11) + 1) * 0x1p-53;
    out[i] = (float)(1.0 / uu);
  }
}

// Embedding rows of tokens[n]: q [n][Hq][D], k/v [n][Hkv][D], bf16.
__global__ void embed_kernel(uint64_t seed, const int32_t* tokens, int n, int Hq, int Hkv, int D,
                             const float* key_mult, uint16_t* q, uint16_t* k, uint16_t* v) {
  const uint64_t key = splitmix64(seed);
  const int i = blockIdx.x;
  if (i >= n) return;
  const uint64_t tok = (uint64_t)(uint32_t)tokens[i];
  for (int e = threadIdx.x; e < (Hq + 2 * Hkv) * D; e += blockDim.x) {
    const int d = e % D, hh = e / D;
    if (hh < Hq) {
      q[((size_t)i * Hq + hh) * D + d] = bf16_rne(z_fp32(draw(key, kRoleEmbQ, (tok << 32) | ((uint64_t)hh << 16) | d)));
    } else if (hh < Hq + Hkv) {
      const int h = hh - Hq;
      uint16_t x = bf16_rne(z_fp32(draw(key, kRoleEmbK, (tok << 32) | ((uint64_t)h << 16) | d)));
      if (key_mult != nullptr) x = bf16_rne(__uint_as_float((uint32_t)x << 16) * key_mult[h * D + d]);
      k[((size_t)i * Hkv + h) * D + d] = x;
    } else {
      const int h = hh - Hq - Hkv;
      v[((size_t)i * Hkv + h) * D + d] = bf16_rne(z_fp32(draw(key, kRoleEmbV, (tok << 32) | ((uint64_t)h << 16) | d)));
    }
  }
}

// Draft-step embedding: token of sequence b is tokens[b * stride]; writes q
// [B][Hq][D] (bf16) and appends k, v at row tail_len[b] of the tail
// ([B][Hkv][tail_cap][D], fp16 or bf16), then increments tail_len[b]. A full
// tail is left unchanged.
__global__ void embed_draft_kernel(uint64_t seed, const int32_t* tokens, int stride, int Hq, int Hkv, int D,
                                   const float* key_mult, uint16_t* q, uint16_t* tail_k, uint16_t* tail_v,
                                   int tail_cap, int tail_fp16, int32_t* tail_len) {
  const uint64_t key = splitmix64(seed);
  const int b = blockIdx.x;
  const uint64_t tok = (uint64_t)(uint32_t)tokens[(size_t)b * stride];
  const int row = tail_len[b];
  const bool room = row >= 0 && row < tail_cap;
  for (int e = threadIdx.x; e < (Hq + 2 * Hkv) * D; e += blockDim.x) {
    const int d = e % D, hh = e / D;
    if (hh < Hq) {
      q[((size_t)b * Hq + hh) * D + d] = bf16_rne(z_fp32(draw(key, kRoleEmbQ, (tok << 32) | ((uint64_t)hh << 16) | d)));
    } else if (room && hh < Hq + Hkv) {
      const int h = hh - Hq;
      uint16_t x = bf16_rne(z_fp32(draw(key, kRoleEmbK, (tok << 32) | ((uint64_t)h << 16) | d)));
      float xf = __uint_as_float((uint32_t)x << 16);
      if (key_mult != nullptr) xf = __uint_as_float((uint32_t)bf16_rne(xf * key_mult[h * D + d]) << 16);
      tail_k[(((size_t)b * Hkv + h) * tail_cap + row) * D + d] = to_out(xf, tail_fp16);
    } else if (room) {
      const int h = hh - Hq - Hkv;
      const uint16_t x = bf16_rne(z_fp32(draw(key, kRoleEmbV, (tok << 32) | ((uint64_t)h << 16) | d)));
      tail_v[(((size_t)b * Hkv + h) * tail_cap + row) * D + d] = to_out(__uint_as_float((uint32_t)x << 16), tail_fp16);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && room) tail_len[b] = row + 1;
}

unsigned grid_for(size_t n) {
  const size_t g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

extern "C" {

int vcs_fill_ctx(uint64_t seed, int which_v, int B, int Hkv, int T, int D, int t_cap, const float* key_mult,
                 void* out, hipStream_t s) {
  if (T > t_cap || T < 0) return -1;
  hipLaunchKernelGGL(fill_ctx_kernel, dim3(grid_for((size_t)B * Hkv * T * D)), dim3(256), 0, s, seed,
                     which_v ? kRoleCtxV : kRoleCtxK, B, Hkv, T, D, t_cap, which_v ? nullptr : key_mult,
                     static_cast<uint16_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int vcs_fill_w(uint64_t seed, int V, int H, void* out, hipStream_t s) {
  hipLaunchKernelGGL(fill_w_kernel, dim3(grid_for((size_t)V * H)), dim3(256), 0, s, seed, V, H,
                     static_cast<uint16_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int vcs_fill_scores(uint64_t seed, int B, int Hkv, int T, float* out, hipStream_t s) {
  hipLaunchKernelGGL(fill_scores_kernel, dim3(grid_for((size_t)B * Hkv * T)), dim3(256), 0, s, seed, B, Hkv, T, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int vcs_embed(uint64_t seed, const int32_t* tokens, int n, int Hq, int Hkv, int D, const float* key_mult, void* q,
              void* k, void* v, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(embed_kernel, dim3(n), dim3(256), 0, s, seed, tokens, n, Hq, Hkv, D, key_mult,
                     static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), static_cast<uint16_t*>(v));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int vcs_embed_draft(uint64_t seed, const int32_t* tokens, int stride, int B, int Hq, int Hkv, int D,
                    const float* key_mult, void* q, void* tail_k, void* tail_v, int tail_cap, int tail_fp16,
                    int32_t* tail_len, hipStream_t s) {
  hipLaunchKernelGGL(embed_draft_kernel, dim3(B), dim3(256), 0, s, seed, tokens, stride, Hq, Hkv, D, key_mult,
                     static_cast<uint16_t*>(q), static_cast<uint16_t*>(tail_k), static_cast<uint16_t*>(tail_v),
                     tail_cap, tail_fp16, tail_len);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
