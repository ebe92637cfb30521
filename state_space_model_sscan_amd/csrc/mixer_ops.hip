// mixer_ops.hip -- the steps next to the scan: causal depthwise conv1d + silu in
// front of it, and the gated RMS norm after the Mamba-2 SSD. Both are streams
// over HBM with a few flops per byte, so the kernels are shaped for wide,
// coalesced accesses: a lane moves 16 bytes of a token row per access.
//
// conv1d + silu ("Mamba-2", nnterp encyclopedia, section "The block, in order":
// x, B, C = silu(conv1d(xBC)), causal, width 4; "Mamba", tokentrails lineage,
// section "Code": depthwise, width 4): a lane owns 16 bytes of channels (8 bf16
// or 4 fp32) and walks a run of tokens, four rows in flight at a time, with the
// last W-1 inputs in registers; the W-1 inputs before the run come from x itself
// or, before the call's first token, from the carried conv state. Neighbouring
// lanes take neighbouring channel groups, so a wave reads whole 1 KiB row
// pieces. Widths that do not split into 16-byte groups take a lane per channel.
//
// gated RMS norm ("Mamba-2", section "The block, in order" and the note under
// it): g = y * silu(z) normalised over the whole width of the row, times the
// norm's weight. One workgroup per row holds its g in registers (16-byte loads
// of y and z), sums g^2 (wave reduction, then across the 4 waves in LDS) and
// writes g * rsqrt(mean + eps) * weight. Rows too wide for the registers, or
// not a whole number of 16-byte groups, re-read the L2-hot row instead.
#include "device_common.hpp"
#include "mixer_ops.hpp"

namespace sscan {

namespace {

constexpr int kConvTokens = 64;

template <typename T, int W>
__global__ __launch_bounds__(256) void conv1d_silu_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.Dc) return;
  const int64_t b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.y * kConvTokens;
  const int64_t t1 = min(a.L, t0 + kConvTokens);
  const T* x = (const T*)a.x;
  T* out = (T*)a.out;
  float wt[W];
#pragma unroll
  for (int kk = 0; kk < W; ++kk) wt[kk] = a.weight[c * W + kk];
  const float bias = a.bias ? a.bias[c] : 0.0f;
  float hist[W > 1 ? W - 1 : 1];  // inputs at t0-W+1 .. t0-1, oldest first
#pragma unroll
  for (int kk = 0; kk < W - 1; ++kk) {
    const int64_t pos = t0 - (W - 1) + kk;
    if (pos >= 0)
      hist[kk] = Act<T>::ld(x + (b * a.L + pos) * a.Dc + c);
    else
      hist[kk] = a.state_in ? a.state_in[(b * a.Dc + c) * (W - 1) + (W - 1 + pos)] : 0.0f;
  }
  for (int64_t t = t0; t < t1; ++t) {
    const float xt = Act<T>::ld(x + (b * a.L + t) * a.Dc + c);
    float acc = bias;
#pragma unroll
    for (int kk = 0; kk < W - 1; ++kk) acc = fmaf(wt[kk], hist[kk], acc);
    acc = fmaf(wt[W - 1], xt, acc);
    Act<T>::st(out + (b * a.L + t) * a.Dc + c, silu(acc));
#pragma unroll
    for (int kk = 0; kk + 1 < W - 1; ++kk) hist[kk] = hist[kk + 1];
    if (W > 1) hist[W > 1 ? W - 2 : 0] = xt;
  }
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16 bytes of a row as fp32 values: 4 fp32 or 8 bf16 (little-endian pairs).
// Stores are non-temporal: the outputs are not read again by these kernels
// (measured 3-4% faster on both streams).
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void ld(const float* p, float* v) {
    const v4u r = *(const v4u*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
  }
  static __device__ __forceinline__ void st(float* p, const float* v) {
    __builtin_nontemporal_store(v4u{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}, (v4u*)p);
  }
};
template <> struct Vec16<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void ld(const uint16_t* p, float* v) {
    const v4u r = *(const v4u*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(uint16_t* p, const float* v) {
    v4u r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    __builtin_nontemporal_store(r, (v4u*)p);
  }
};

constexpr int kConvUnroll = 4;  // token rows a lane has in flight

// One lane: channels [c0, c0 + V) of batch row b, tokens [t0, t0 + tpl). The
// sum for an output is formed in the order bias, w_0 x_{t-W+1}, ..., w_{W-1} x_t,
// as in conv1d_silu_kernel, so both kernels give the same bits.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv1d_silu_vec_kernel(ConvArgs a, int64_t tpl, int64_t ntb) {
  constexpr int V = Vec16<T>::n;
  constexpr int U = kConvUnroll;
  const int64_t nvec = a.Dc / V;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cv = gid % nvec, rest = gid / nvec;
  const int64_t tb = rest % ntb, b = rest / ntb;
  if (b >= a.batch) return;
  const int64_t c0 = cv * V;
  const int64_t t0 = tb * tpl, t1 = min(a.L, t0 + tpl);
  const T* xp = (const T*)a.x + b * a.L * a.Dc + c0;
  T* op = (T*)a.out + b * a.L * a.Dc + c0;
  float wt[W][V], bias[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
#pragma unroll
    for (int kk = 0; kk < W; ++kk) wt[kk][j] = a.weight[(c0 + j) * W + kk];
    bias[j] = a.bias ? a.bias[c0 + j] : 0.0f;
  }
  // win[0 .. W-2]: the inputs at t-W+1 .. t-1; win[W-1 ..]: the rows in flight
  float win[W - 1 + U][V];
#pragma unroll
  for (int kk = 0; kk < W - 1; ++kk) {
    const int64_t pos = t0 - (W - 1) + kk;
    if (pos >= 0) {
      Vec16<T>::ld(xp + pos * a.Dc, win[kk]);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j)
        win[kk][j] = a.state_in ? a.state_in[(b * a.Dc + c0 + j) * (W - 1) + (W - 1 + pos)] : 0.0f;
    }
  }
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) Vec16<T>::ld(xp + (t + u) * a.Dc, win[W - 1 + u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        float acc = bias[j];
#pragma unroll
        for (int kk = 0; kk < W; ++kk) acc = fmaf(wt[kk][j], win[u + kk][j], acc);
        o[j] = silu(acc);
      }
      Vec16<T>::st(op + (t + u) * a.Dc, o);
    }
#pragma unroll
    for (int kk = 0; kk < W - 1; ++kk)
#pragma unroll
      for (int j = 0; j < V; ++j) win[kk][j] = win[U + kk][j];
  }
  for (; t < t1; ++t) {
    Vec16<T>::ld(xp + t * a.Dc, win[W - 1]);
    float o[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float acc = bias[j];
#pragma unroll
      for (int kk = 0; kk < W; ++kk) acc = fmaf(wt[kk][j], win[kk][j], acc);
      o[j] = silu(acc);
    }
    Vec16<T>::st(op + t * a.Dc, o);
#pragma unroll
    for (int kk = 0; kk < W - 1; ++kk)
#pragma unroll
      for (int j = 0; j < V; ++j) win[kk][j] = win[kk + 1][j];
  }
}

// conv_state_out = the last W-1 inputs of [state_in, x] (oldest first).
template <typename T>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.Dc) return;
  const int64_t b = blockIdx.y;
  const int W = (int)a.W;
  const T* x = (const T*)a.x;
  for (int kk = 0; kk < W - 1; ++kk) {
    const int64_t pos = a.L - (W - 1) + kk;
    float v;
    if (pos >= 0)
      v = Act<T>::ld(x + (b * a.L + pos) * a.Dc + c);
    else
      v = a.state_in ? a.state_in[(b * a.Dc + c) * (W - 1) + (W - 1 + pos)] : 0.0f;
    a.state_out[(b * a.Dc + c) * (W - 1) + kk] = v;
  }
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* y = (const T*)a.y + row * a.width;
  const T* z = (const T*)a.z + row * a.width;
  T* out = (T*)a.out + row * a.width;
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < a.width; i += 256) {
    const float g = Act<T>::ld(y + i) * silu(Act<T>::ld(z + i));
    ss = fmaf(g, g, ss);
  }
  const float total = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(total / (float)a.width + a.eps);
  for (int64_t i = threadIdx.x; i < a.width; i += 256) {
    const float g = Act<T>::ld(y + i) * silu(Act<T>::ld(z + i));
    Act<T>::st(out + i, g * inv * a.weight[i]);
  }
}

// Row held in registers: thread i owns the 16-byte groups i, i + 256, ...
template <typename T, int VPL>
__global__ __launch_bounds__(256) void gated_rmsnorm_vec_kernel(NormArgs a) {
  constexpr int V = Vec16<T>::n;
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nvec = (int)(a.width / V);
  const T* y = (const T*)a.y + row * a.width;
  const T* z = (const T*)a.z + row * a.width;
  T* out = (T*)a.out + row * a.width;
  float g[VPL][V];
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < nvec) {
      float zv[V];
      Vec16<T>::ld(y + (int64_t)i * V, g[k]);
      Vec16<T>::ld(z + (int64_t)i * V, zv);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        g[k][j] *= silu(zv[j]);
        ss = fmaf(g[k][j], g[k][j], ss);
      }
    }
  }
  const float total = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(total / (float)a.width + a.eps);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < nvec) {
      float wv[V], o[V];
      Vec16<float>::ld(a.weight + (int64_t)i * V, wv);
      if (V == 8) Vec16<float>::ld(a.weight + (int64_t)i * V + 4, wv + 4);
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = g[k][j] * inv * wv[j];
      Vec16<T>::st(out + (int64_t)i * V, o);
    }
  }
}

// Tokens per lane for the vector kernel: the longest run (fewer re-read history
// rows) that still gives about 8 waves per SIMD.
int64_t conv_tokens_per_lane(int64_t lanes_per_run_block, int64_t L) {
  int64_t tpl = 128;
  while (tpl > 16 && lanes_per_run_block * ((L + tpl - 1) / tpl) < 256 * 4 * 8 * 64) tpl >>= 1;
  return tpl;
}

template <typename T, int W>
void launch_conv_vec(const ConvArgs& a, hipStream_t s) {
  const int64_t nvec = a.Dc / Vec16<T>::n;
  const int64_t tpl = conv_tokens_per_lane(a.batch * nvec, a.L);
  const int64_t ntb = (a.L + tpl - 1) / tpl;
  const int64_t lanes = a.batch * ntb * nvec;
  hipLaunchKernelGGL((conv1d_silu_vec_kernel<T, W>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, a,
                     tpl, ntb);
}

template <typename T>
void launch_conv_t(const ConvArgs& a, hipStream_t s) {
  const unsigned cb = (unsigned)((a.Dc + 255) / 256);
  if (a.L > 0) {
    const int64_t vec_lanes = a.batch * ((a.L + 15) / 16) * (a.Dc / Vec16<T>::n);
    if (a.Dc % Vec16<T>::n == 0 && a.W >= 2 && a.W <= 4 && vec_lanes / 256 < (int64_t(1) << 30)) {
      switch (a.W) {
        case 2: launch_conv_vec<T, 2>(a, s); break;
        case 3: launch_conv_vec<T, 3>(a, s); break;
        default: launch_conv_vec<T, 4>(a, s); break;
      }
    } else {
      const dim3 grid(cb, (unsigned)((a.L + kConvTokens - 1) / kConvTokens), (unsigned)a.batch);
      switch (a.W) {
        case 1: hipLaunchKernelGGL((conv1d_silu_kernel<T, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((conv1d_silu_kernel<T, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((conv1d_silu_kernel<T, 3>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((conv1d_silu_kernel<T, 4>), grid, dim3(256), 0, s, a); break;
        case 5: hipLaunchKernelGGL((conv1d_silu_kernel<T, 5>), grid, dim3(256), 0, s, a); break;
        case 6: hipLaunchKernelGGL((conv1d_silu_kernel<T, 6>), grid, dim3(256), 0, s, a); break;
        case 7: hipLaunchKernelGGL((conv1d_silu_kernel<T, 7>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((conv1d_silu_kernel<T, 8>), grid, dim3(256), 0, s, a); break;
      }
    }
  }
  if (a.state_out && a.W > 1)
    hipLaunchKernelGGL(conv_state_kernel<T>, dim3(cb, (unsigned)a.batch), dim3(256), 0, s, a);
}

template <typename T>
void launch_norm_t(const NormArgs& a, hipStream_t s) {
  constexpr int V = Vec16<T>::n;
  const dim3 grid((unsigned)a.rows);
  const int64_t nvec = a.width / V;
  if (a.width % V != 0 || nvec > 256 * 8) {
    hipLaunchKernelGGL(gated_rmsnorm_kernel<T>, grid, dim3(256), 0, s, a);
  } else if (nvec <= 256) {
    hipLaunchKernelGGL((gated_rmsnorm_vec_kernel<T, 1>), grid, dim3(256), 0, s, a);
  } else if (nvec <= 512) {
    hipLaunchKernelGGL((gated_rmsnorm_vec_kernel<T, 2>), grid, dim3(256), 0, s, a);
  } else if (nvec <= 1024) {
    hipLaunchKernelGGL((gated_rmsnorm_vec_kernel<T, 4>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((gated_rmsnorm_vec_kernel<T, 8>), grid, dim3(256), 0, s, a);
  }
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.bf16) launch_conv_t<uint16_t>(a, s);
  else launch_conv_t<float>(a, s);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16) launch_norm_t<uint16_t>(a, s);
  else launch_norm_t<float>(a, s);
  return hipGetLastError();
}

}  // namespace sscan
