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
#include "common.h"

namespace vsa {

namespace {

constexpr float kE4M3Max = 448.f;

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

// Q or K: one workgroup per (b, h, cube).  Reads the cube's raster rows,
// reduces the block maximum, writes the codes as token-major rows
// [B, H, Np, D] (bytes) and the scale [B, H, Nc].
template <int D>
__global__ void __launch_bounds__(256) quant_cube(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                  float* __restrict__ scale, KGeom g) {
  constexpr int CH = D / 8;             // 16-byte bf16 chunks per row
  constexpr int PER = 64 * CH / 256;    // chunks per thread
  __shared__ float red[256 / 64];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  uint4 v[PER];
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int f = threadIdx.x + 256 * k, l = f / CH, ch = f % CH;
    const long long tok = cube_token(g, ct, cy, cx, l);
    v[k] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v[k] = reinterpret_cast<const uint4*>(x + (((long long)b * g.S + tok) * g.H + h) * D)[ch];
    const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf_lo(w4[e])), fabsf(bf_hi(w4[e]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = inv_of(m);
  const long long row0 = ((long long)b * g.H + h) * g.Np + 64LL * c;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int f = threadIdx.x + 256 * k, l = f / CH, ch = f % CH;
    const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    const uint32_t lo = to_e4m3x4(bf_lo(w4[0]) * inv, bf_hi(w4[0]) * inv, bf_lo(w4[1]) * inv, bf_hi(w4[1]) * inv);
    const uint32_t hi = to_e4m3x4(bf_lo(w4[2]) * inv, bf_hi(w4[2]) * inv, bf_lo(w4[3]) * inv, bf_hi(w4[3]) * inv);
    *reinterpret_cast<uint2*>(x8 + (row0 + l) * D + 8 * ch) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scale[((long long)b * g.H + h) * g.nc + c] = __fdiv_rn(m, kE4M3Max);
}

// V, pass 1: per (b, h, cube) the largest |v| of every channel -> cmax [B, H, Nc, D].
template <int D>
__global__ void __launch_bounds__(256) chan_max_cube(const uint16_t* __restrict__ x, float* __restrict__ cmax,
                                                     KGeom g) {
  constexpr int CH = D / 8;
  __shared__ float part[256 / CH][D];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const int ch = threadIdx.x % CH, r0 = threadIdx.x / CH;  // rows r0, r0 + 256/CH, ...
  float m[8] = {};
  for (int l = r0; l < 64; l += 256 / CH) {
    const long long tok = cube_token(g, ct, cy, cx, l);
    if (tok < 0) continue;
    const uint4 v = reinterpret_cast<const uint4*>(x + (((long long)b * g.S + tok) * g.H + h) * D)[ch];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] = fmaxf(m[2 * e], fabsf(bf_lo(w4[e])));
      m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(bf_hi(w4[e])));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][8 * ch + e] = m[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float r = 0.f;
    for (int k = 0; k < 256 / CH; ++k) r = fmaxf(r, part[k][threadIdx.x]);
    cmax[(((long long)b * g.H + h) * g.nc + c) * D + threadIdx.x] = r;
  }
}

// V, pass 2: per (b, h) the channel maxima over all cubes -> scale [B, H, D].
__global__ void __launch_bounds__(256) chan_max_head(const float* __restrict__ cmax, float* __restrict__ vmax,
                                                     float* __restrict__ scale, KGeom g) {
  const long long bh = blockIdx.x;
  for (int d = threadIdx.x; d < g.D; d += 256) {
    float r = 0.f;
    for (int c = 0; c < g.nc; ++c) r = fmaxf(r, cmax[(bh * g.nc + c) * g.D + d]);
    vmax[bh * g.D + d] = r;
    scale[bh * g.D + d] = __fdiv_rn(r, kE4M3Max);
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

// V, pass 3: per (b, h, cube) codes of v * (448 / vmax[channel]), stored as
// the cube transposed: [B, H, Nc, D, 64] bytes, keys in vkey_pos order.
template <int D>
__global__ void __launch_bounds__(256) quant_v(const uint16_t* __restrict__ x, const float* __restrict__ vmax,
                                               uint8_t* __restrict__ v8t, KGeom g) {
  constexpr int CH = D / 8;
  __shared__ uint8_t tile[D][64 + 4];  // [channel][key position], padded rows
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * g.H + h;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  for (int f = threadIdx.x; f < 64 * CH; f += 256) {
    const int l = f / CH, ch = f % CH;
    const long long tok = cube_token(g, ct, cy, cx, l);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v = reinterpret_cast<const uint4*>(x + (((long long)b * g.S + tok) * g.H + h) * D)[ch];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    const int pos = vkey_pos(l);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d0 = 8 * ch + 2 * e;
      const float a = bf_lo(w4[e]) * inv_of(vmax[bh * D + d0]);
      const float bb = bf_hi(w4[e]) * inv_of(vmax[bh * D + d0 + 1]);
      const uint32_t w = to_e4m3x4(a, bb, 0.f, 0.f);
      tile[d0][pos] = (uint8_t)(w & 0xFF);
      tile[d0 + 1][pos] = (uint8_t)((w >> 8) & 0xFF);
    }
  }
  __syncthreads();
  // D rows of 64 bytes: 4 x 16 bytes per row.
  uint8_t* out = v8t + (bh * g.nc + c) * (long long)D * 64;
  for (int f = threadIdx.x; f < D * 4; f += 256) {
    const int d = f >> 2, q = f & 3;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[d][16 * q + 4 * e] | ((uint32_t)tile[d][16 * q + 4 * e + 1] << 8) |
             ((uint32_t)tile[d][16 * q + 4 * e + 2] << 16) | ((uint32_t)tile[d][16 * q + 4 * e + 3] << 24);
    *reinterpret_cast<uint4*>(out + d * 64 + 16 * q) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

size_t quant_v_workspace_bytes(const KGeom& g) {
  return (size_t)g.B * g.H * ((size_t)g.nc + 1) * g.D * sizeof(float);
}

hipError_t launch_quant_qk(const KGeom& g, const uint16_t* x, uint8_t* x8, float* scale, hipStream_t s) {
  const dim3 grid(g.nc, g.H, g.B);
  if (g.D == 64) quant_cube<64><<<grid, dim3(256), 0, s>>>(x, x8, scale, g);
  else quant_cube<128><<<grid, dim3(256), 0, s>>>(x, x8, scale, g);
  return hipGetLastError();
}

hipError_t launch_quant_v(const KGeom& g, const uint16_t* x, uint8_t* v8t, float* scale, void* ws, hipStream_t s) {
  float* cmax = static_cast<float*>(ws);
  float* vmax = cmax + (size_t)g.B * g.H * g.nc * g.D;
  const dim3 grid(g.nc, g.H, g.B);
  if (g.D == 64) chan_max_cube<64><<<grid, dim3(256), 0, s>>>(x, cmax, g);
  else chan_max_cube<128><<<grid, dim3(256), 0, s>>>(x, cmax, g);
  chan_max_head<<<dim3(g.B * g.H), dim3(256), 0, s>>>(cmax, vmax, scale, g);
  if (g.D == 64) quant_v<64><<<grid, dim3(256), 0, s>>>(x, vmax, v8t, g);
  else quant_v<128><<<grid, dim3(256), 0, s>>>(x, vmax, v8t, g);
  return hipGetLastError();
}

}  // namespace vsa
