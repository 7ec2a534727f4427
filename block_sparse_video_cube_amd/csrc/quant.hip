// 8-bit (fp8 E4M3) inputs of the low-precision fine stage.
//
// SageAttention and SageAttention2 run the key matrix products of attention
// at 8 bits or lower, and sparsity composes with such low-bit matrix cores
// (TurboDiffusion article, section "稀疏、蒸馏与全链路量化").  Here the
// format is OCP E4M3 (bias 7, largest finite 448, as gfx950's
// v_cvt_pk_fp8_f32 and fp8 MFMAs use it); Q and K get one scale per
// (b, h, cube), V one per (b, h, channel) over the whole head, so that the
// per-channel scale of V can be taken out of the sum over key cubes.
//
// Exact fp32 steps (the same on every path that checks them):
//   m = largest |x| of the block over valid tokens, inv = 448 / m (0 if m = 0),
//   q = clamp(x * inv, -448, 448), code = E4M3 round-to-nearest-even of q,
//   stored scale = m / 448 (dequantized value = code * scale).
//
// Two passes over raster [B, S, H, D] inputs (HBM bound):
//   pass 1, one workgroup per (b, h, cube): Q and K codes and scales, and
//     optionally their cube means (the coarse stage's pooled Q and K, summed
//     in the same order as the pooling kernel, so bit-identical to it); V's
//     per-channel maxima over the cube, folded into the head maxima with
//     atomic max on the fp32 bit patterns (non-negative floats order as
//     unsigned integers);
//   pass 2, one workgroup per (b, h, cube): V's codes, transposed per cube.
#include <mutex>

#include "common.h"

namespace vsa {

namespace {

constexpr float kE4M3Max = 448.f;
constexpr int kQThreads = 256;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four fp32 values (already scaled) -> four E4M3 codes in one word.
__device__ __forceinline__ uint32_t to_e4m3x4(float a, float b, float c, float d) {
  const auto cl = [](float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float inv_of(float m) { return m > 0.f ? __fdiv_rn(kE4M3Max, m) : 0.f; }

// Raster token of local row l of cube (ct, cy, cx), or -1 for a padded token.
__device__ __forceinline__ long long cube_token(const KGeom& g, int ct, int cy, int cx, int l) {
  const int t = 4 * ct + (l >> 4), y = 4 * cy + ((l >> 2) & 3), x = 4 * cx + (l & 3);
  if (t >= g.T || y >= g.Hg || x >= g.W) return -1;
  return ((long long)t * g.Hg + y) * g.W + x;
}

// The cube's rows of one head: thread t holds 16-byte chunk t % (D / 8) of
// rows t / (D / 8) + 256 k / (D / 8), zeros for padded tokens.
template <int D>
struct CubeRows {
  static constexpr int CH = D / 8;
  static constexpr int PER = 64 * CH / kQThreads;
  uint4 x[PER];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, const KGeom& g, int b, int h, int ct, int cy,
                                       int cx) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int f = threadIdx.x + kQThreads * k, l = f / CH, ch = f % CH;
      const long long tok = cube_token(g, ct, cy, cx, l);
      x[k] = make_uint4(0, 0, 0, 0);
      if (tok >= 0) x[k] = reinterpret_cast<const uint4*>(src + (((long long)b * g.S + tok) * g.H + h) * D)[ch];
    }
  }
};

// Largest |x| over the workgroup (all threads get it).  red: 4 floats of LDS.
__device__ __forceinline__ float block_max(float m, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Q or K of one cube: codes [B, H, Np, D] bytes, scale [B, H, Nc], and the
// cube mean over valid tokens when mean != nullptr.  The mean is summed as
// the pooling kernel sums it: per thread over its rows in order, then across
// the threads of a chunk by exchanges at lane distances D/8 .. 32, then the
// four wavefronts in order, divided by the count of valid tokens.  (Padded
// rows hold zeros here; adding +0 to the fp32 sums changes no bit.)
template <int D, bool COMPACT>
__device__ __forceinline__ void quant_block(const CubeRows<D>& r, uint8_t* __restrict__ x8,
                                            float* __restrict__ scale, float* __restrict__ mean, const KGeom& g,
                                            long long bh, int c, int ct, int cy, int cx, int count, float* red,
                                            float (*part)[D]) {
  constexpr int CH = D / 8, PER = CubeRows<D>::PER;
  float m = 0.f;
  float acc[8] = {};
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const uint32_t w4[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf_lo(w4[e]), hi = bf_hi(w4[e]);
      m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
      acc[2 * e] += lo;
      acc[2 * e + 1] += hi;
    }
  }
  m = block_max(m, red);
  const float inv = inv_of(m);
  const long long row0 = bh * g.Np + 64LL * c;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int f = threadIdx.x + kQThreads * k, l = f / CH, ch = f % CH;
    const uint32_t w4[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
    const uint32_t lo = to_e4m3x4(bf_lo(w4[0]) * inv, bf_hi(w4[0]) * inv, bf_lo(w4[1]) * inv, bf_hi(w4[1]) * inv);
    const uint32_t hi = to_e4m3x4(bf_lo(w4[2]) * inv, bf_hi(w4[2]) * inv, bf_lo(w4[3]) * inv, bf_hi(w4[3]) * inv);
    const int rr = COMPACT ? compact_row(g, ct, cy, cx, l) : l;
    *reinterpret_cast<uint2*>(x8 + (row0 + rr) * D + 8 * ch) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scale[bh * g.nc + c] = __fdiv_rn(m, kE4M3Max);
  if (mean == nullptr) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = CH; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < CH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[w][lane * 8 + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
#pragma unroll
    for (int rr = 0; rr < kQThreads / 64; ++rr) sum += part[rr][threadIdx.x];
    mean[(bh * g.nc + c) * D + threadIdx.x] = sum / (float)count;
  }
}

// Pass 1.  vmax: [B, H, D] fp32 bit patterns, zero on entry.  KCOMPACT: the
// K codes go to compact cube-major rows (the packed fp8 stage's layout).
template <int D, bool KCOMPACT>
__global__ void __launch_bounds__(kQThreads) quant_pass1(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint8_t* __restrict__ q8,
                                                          float* __restrict__ qscale, float* __restrict__ qmean,
                                                          uint8_t* __restrict__ k8, float* __restrict__ kscale,
                                                          float* __restrict__ kmean, uint32_t* __restrict__ vmax,
                                                          KGeom g) {
  constexpr int CH = D / 8, PER = CubeRows<D>::PER;
  __shared__ float red[2][kQThreads / 64];
  __shared__ float part[3][kQThreads / 64][D];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * g.H + h;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  CubeRows<D> rq, rk, rv;
  rq.load(q, g, b, h, ct, cy, cx);
  rk.load(k, g, b, h, ct, cy, cx);
  rv.load(v, g, b, h, ct, cy, cx);
  const int count = cube_count(g, ct, cy, cx);
  quant_block<D, false>(rq, q8, qscale, qmean, g, bh, c, ct, cy, cx, count, red[0], part[0]);
  quant_block<D, KCOMPACT>(rk, k8, kscale, kmean, g, bh, c, ct, cy, cx, count, red[1], part[1]);
  // V: largest |v| of every channel over the cube's rows.
  float cm[8] = {};
#pragma unroll
  for (int kk = 0; kk < PER; ++kk) {
    const uint32_t w4[4] = {rv.x[kk].x, rv.x[kk].y, rv.x[kk].z, rv.x[kk].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cm[2 * e] = fmaxf(cm[2 * e], fabsf(bf_lo(w4[e])));
      cm[2 * e + 1] = fmaxf(cm[2 * e + 1], fabsf(bf_hi(w4[e])));
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = CH; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) cm[e] = fmaxf(cm[e], __shfl_xor(cm[e], off));
  if (lane < CH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[2][w][lane * 8 + e] = cm[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float r = part[2][0][threadIdx.x];
#pragma unroll
    for (int rr = 1; rr < kQThreads / 64; ++rr) r = fmaxf(r, part[2][rr][threadIdx.x]);
    atomicMax(vmax + bh * D + threadIdx.x, __float_as_uint(r));
  }
}

// Position of key k (0..63) inside a row of the fp8 V^T tile: the order in
// which the fp8 fine stage's accumulator hands P to the next product, so that
// lane half h finds its 32 keys contiguous.  k = 32 t + 16 g + 8 h + e sits at
// 32 h + 16 t + 8 g + e.
__device__ __forceinline__ int vkey_pos(int k) {
  const int t = k >> 5, gg = (k >> 4) & 1, hh = (k >> 3) & 1, e = k & 7;
  return 32 * hh + 16 * t + 8 * gg + e;
}

// Pass 2: codes of v * (448 / vmax[channel]) stored as the cube transposed,
// [B, H, Nc, D, 64] bytes with keys in vkey_pos order, or (SLOTS, the packed
// fp8 stage's layout) [B, H, Nc, 4, D, 16]: the cube's keys in compact order
// cut into four 16-key slots, each transposed; cube 0's workgroup also writes
// the scales [B, H, D].
template <int D, bool SLOTS>
__global__ void __launch_bounds__(kQThreads) quant_pass2(const uint16_t* __restrict__ v,
                                                          const uint32_t* __restrict__ vmax,
                                                          uint8_t* __restrict__ v8t, float* __restrict__ vscale,
                                                          KGeom g) {
  constexpr int CH = D / 8, PER = CubeRows<D>::PER, LD = 68;  // LDS row: 64 key bytes + 4
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * LD];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * g.H + h;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  CubeRows<D> rv;
  rv.load(v, g, b, h, ct, cy, cx);
  const int ch = threadIdx.x % CH;  // the same chunk (8 channels) on every row of this thread
  float inv[8];
  {
    const uint4 m0 = reinterpret_cast<const uint4*>(vmax + bh * D)[2 * ch];
    const uint4 m1 = reinterpret_cast<const uint4*>(vmax + bh * D)[2 * ch + 1];
    const uint32_t mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = inv_of(__uint_as_float(mm[e]));
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int f = threadIdx.x + kQThreads * k, l = f / CH;
    const int pos = SLOTS ? compact_row(g, ct, cy, cx, l) : vkey_pos(l);
    const uint32_t w4[4] = {rv.x[k].x, rv.x[k].y, rv.x[k].z, rv.x[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t wd = to_e4m3x4(bf_lo(w4[e]) * inv[2 * e], bf_hi(w4[e]) * inv[2 * e + 1], 0.f, 0.f);
      tile[(8 * ch + 2 * e) * LD + pos] = (uint8_t)(wd & 0xFF);
      tile[(8 * ch + 2 * e + 1) * LD + pos] = (uint8_t)((wd >> 8) & 0xFF);
    }
  }
  __syncthreads();
  uint8_t* out = v8t + (bh * g.nc + c) * (long long)D * 64;
  for (int f = threadIdx.x; f < D * 4; f += kQThreads) {
    const int d = f >> 2, qq = f & 3;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + d * LD + 16 * qq);
    // SLOTS: bytes 16 qq .. +15 of row d are keys 0..15 of slot qq.
    *reinterpret_cast<uint4*>(out + (SLOTS ? (qq * D + d) * 16 : d * 64 + 16 * qq)) =
        make_uint4(src[0], src[1], src[2], src[3]);
  }
  if (c == 0 && threadIdx.x < D)
    vscale[bh * D + threadIdx.x] = __fdiv_rn(__uint_as_float(vmax[bh * D + threadIdx.x]), kE4M3Max);
}

__global__ void __launch_bounds__(kQThreads) zero_words(uint32_t* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * kQThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kQThreads)
    p[i] = 0u;
}

template <int D>
void launch_quant_t(const KGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8, float* qs,
                    uint8_t* k8, float* ks, uint8_t* v8t, float* vs, float* qmean, float* kmean, uint32_t* vmax,
                    bool packed, hipStream_t s) {
  const long long nmax = (long long)g.B * g.H * D;
  zero_words<<<dim3((unsigned)((nmax + kQThreads - 1) / kQThreads)), dim3(kQThreads), 0, s>>>(vmax, nmax);
  const dim3 grid(g.nc, g.H, g.B);
  if (packed) {
    quant_pass1<D, true><<<grid, dim3(kQThreads), 0, s>>>(q, k, v, q8, qs, qmean, k8, ks, kmean, vmax, g);
    quant_pass2<D, true><<<grid, dim3(kQThreads), 0, s>>>(v, vmax, v8t, vs, g);
  } else {
    quant_pass1<D, false><<<grid, dim3(kQThreads), 0, s>>>(q, k, v, q8, qs, qmean, k8, ks, kmean, vmax, g);
    quant_pass2<D, false><<<grid, dim3(kQThreads), 0, s>>>(v, vmax, v8t, vs, g);
  }
}

}  // namespace

// The allocation-free entry point keeps the head maxima of V in this static
// array instead of a caller workspace: every device the library runs on holds
// its own copy (until the process ends).  Host code reaches it only through
// the address hipGetSymbolAddress returns for the device (quant_scratch);
// the array's name is not a device address on the host.
static __device__ __align__(256) uint32_t scratch[VSA_QUANT_SCRATCH_WORDS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint32_t* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t quant_scratch(hipStream_t s, uint32_t** out) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    // Once per device, with that device current.
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

size_t quant_workspace_bytes(const KGeom& g) {
  return ((size_t)g.B * g.H * g.D * sizeof(uint32_t) + 255) / 256 * 256;
}

hipError_t launch_quant(const KGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8,
                        float* qs, uint8_t* k8, float* ks, uint8_t* v8t, float* vs, float* qmean, float* kmean,
                        void* ws, hipStream_t s, bool packed) {
  uint32_t* vmax = static_cast<uint32_t*>(ws);
  if (g.D == 64) launch_quant_t<64>(g, q, k, v, q8, qs, k8, ks, v8t, vs, qmean, kmean, vmax, packed, s);
  else launch_quant_t<128>(g, q, k, v, q8, qs, k8, ks, v8t, vs, qmean, kmean, vmax, packed, s);
  return hipGetLastError();
}

}  // namespace vsa
