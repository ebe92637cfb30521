// ssd_attention.hip -- the SSD scan's hidden attention map as an optional output.
//
// "Mamba-2" (nnterp encyclopedia), section "The hidden attention": per head the
// scan is a causal linear map over tokens, y_t = sum_s alpha[t, s] x_s + D x_t
// before the gate, with
//     alpha[t, s] = (C_t . B_s) * exp(decays_{s+1} + ... + decays_t) * betas_s   (s <= t)
// and 0 above the diagonal; betas = softplus(dt_raw + dt_bias), decays = betas * A,
// A = -exp(A_log) (section "The mixer's values"); head h reads group h / (H / G).
//
// The map is [batch, t, s, heads] fp32: writing it is the whole cost, so the
// work is shaped for the store stream.
//
// attn_prefix_kernel: one workgroup per (batch row, head) forms, in fp64,
//     P[t] = decays_0 + ... + decays_t     (times log2 e)
// and betas_t into the caller's workspace, head-major ([batch, head, token]).
// Each thread sums a contiguous run of tokens, the runs' totals are scanned
// across the workgroup, and each thread then rewalks its run from its offset.
// P is a sum of same-sign terms, so
// exponent(t, s) = P[t] - P[s] = decays_{s+1} + ... + decays_t is exact to
// 2^-53 |P| in fp64, far below the fp32 result.
//
// ssd_attention_kernel: a work item is one batch row, one key tile of 32
// tokens [s0, s0 + 32), one query tile of 32 tokens, and a chunk of at
// most 128 heads (whole groups, or part of one group when a group has more
// than 128 heads). For every query row t of a tile the item writes keys
// s0..s0+31 x the chunk's heads, one contiguous run per row; a lane writes 16
// bytes (4 heads of one key) at a time when the heads per group are a
// multiple of 4, else one value; the stores are marked non-temporal, as the
// map is not read back here. A lane keeps P and betas of its keys in
// registers, the tile's rows of P sit in LDS, and C_t . B_s for the tile comes
// from a small LDS-staged product per group. Query tiles above the key tile
// are zeros; on the diagonal tile the entries with s > t are zeros.
#include <atomic>

#include "device_common.hpp"
#include "mixer_ops.hpp"

namespace sscan {

namespace {

constexpr int kT = 32;        // tokens per tile side
constexpr int kRange = 1;     // query tiles per work item (1 measured best: many short items)
constexpr int kMaxHC = 128;   // heads per chunk
constexpr int kMaxGPC = 8;    // groups per chunk
constexpr int kKC = 64;       // state entries per staging step of C . B
constexpr int kCP = kKC + 1;  // row pitch of the staged C (floats)
constexpr double kLog2eD = 1.4426950408889634;

struct AttnPlan {
  int64_t hpg;     // heads per group
  int64_t HC;      // heads per chunk (the LDS row pitch)
  int64_t GPC;     // groups per chunk (1 when hpg > kMaxHC)
  int64_t cpg;     // chunks per group when hpg > kMaxHC
  int64_t nchunks, nkt, nqr;
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kPrefixBatch = 8;  // dt loads in flight per thread

// One workgroup per (batch row, head): thread i sums the contiguous run of
// tokens [i per, (i + 1) per), the run totals are scanned over the workgroup
// (within each wave, then across the 4 waves through LDS), and each thread
// rewalks its run from its offset, writing P and betas head-major, so that a
// wave's stores are contiguous.
template <typename T>
__global__ __launch_bounds__(256) void attn_prefix_kernel(AttnArgs a) {
  __shared__ double wave_total[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t bh = blockIdx.x;  // batch row * H + head
  const int64_t b = bh / a.H, h = bh % a.H;
  const float A = -expf(a.A_log[h]);
  const float bias = a.dt_bias[h];
  const T* dt = (const T*)a.dt + b * a.L * a.H + h;
  const int64_t per = (a.L + 255) / 256;
  const int64_t lo = min(a.L, tid * per), hi = min(a.L, lo + per);
  double sum = 0.0;
  for (int64_t j0 = lo; j0 < hi; j0 += kPrefixBatch) {
    float bv[kPrefixBatch];
#pragma unroll
    for (int u = 0; u < kPrefixBatch; ++u)
      bv[u] = j0 + u < hi ? softplus(Act<T>::ld(dt + (j0 + u) * a.H) + bias) : 0.0f;
#pragma unroll
    for (int u = 0; u < kPrefixBatch; ++u) sum += (double)bv[u] * (double)A;
  }
  double incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_total[wv] = incl;
  double P = __shfl_up(incl, 1, 64);
  if (lane == 0) P = 0.0;
  __syncthreads();
  for (int q = 0; q < wv; ++q) P += wave_total[q];
  double* wp = a.ws_P + bh * a.L;
  float* wb = a.ws_beta + bh * a.L;
  for (int64_t j0 = lo; j0 < hi; j0 += kPrefixBatch) {
    float bv[kPrefixBatch];
#pragma unroll
    for (int u = 0; u < kPrefixBatch; ++u)
      bv[u] = j0 + u < hi ? softplus(Act<T>::ld(dt + (j0 + u) * a.H) + bias) : 0.0f;
#pragma unroll
    for (int u = 0; u < kPrefixBatch; ++u) {
      P += (double)bv[u] * (double)A;
      if (j0 + u < hi) {
        wp[j0 + u] = P * kLog2eD;
        wb[j0 + u] = bv[u];
      }
    }
  }
}

template <typename T, int VW>
__global__ __launch_bounds__(256) void ssd_attention_kernel(AttnArgs a, AttnPlan p) {
  constexpr int SPT = kT * kMaxHC / VW / 256;  // slots (VW heads of one key) per thread
  extern __shared__ __attribute__((aligned(16))) double smem_d[];
  const int tid = threadIdx.x;
  const int64_t L = a.L, H = a.H, N = a.N;
  int64_t item = blockIdx.x;
  const int64_t qr = item % p.nqr;
  item /= p.nqr;
  const int64_t kt = item % p.nkt;
  item /= p.nkt;
  const int64_t chunk = item % p.nchunks;
  const int64_t b = item / p.nchunks;
  int64_t h_lo, h_hi, g_lo, ngc;
  if (p.hpg <= kMaxHC) {
    h_lo = chunk * p.HC;
    h_hi = min(H, h_lo + p.HC);
    g_lo = h_lo / p.hpg;
    ngc = (h_hi - h_lo) / p.hpg;
  } else {
    const int64_t g = chunk / p.cpg, sub = chunk % p.cpg;
    h_lo = g * p.hpg + sub * kMaxHC;
    h_hi = min(g * p.hpg + p.hpg, h_lo + kMaxHC);
    g_lo = g;
    ngc = 1;
  }
  const int hc = (int)(h_hi - h_lo);
  const int HCp = (int)p.HC;
  const int64_t s0 = kt * kT;
  const int64_t q_first = qr * kRange;
  const int64_t q_end = min(p.nkt, q_first + kRange);

  double* sPq = smem_d;                     // [kT][HCp]: P at the tile's rows
  float* sCB = (float*)(sPq + kT * HCp);    // [GPC][kT (t)][kT (s)]
  float* sC = sCB + p.GPC * kT * kT;        // [kT (t)][kCP]
  float* sB = sC + kT * kCP;                // [kKC][kT (s)]

  const int nslot = kT * hc / VW;
  float* arow = a.alpha + (b * L) * L * H + h_lo;  // + (t * L + s) * H + head offset
  const double* Pb = a.ws_P + (b * H + h_lo) * L;  // [head][token]
  const float* betab = a.ws_beta + (b * H + h_lo) * L;

  double pk[SPT][VW];  // P at the slot's key
  float bt[SPT][VW];   // betas at the slot's key
  int cbi[SPT];        // the slot's column of C . B: group * kT * kT + key
  if (q_end - 1 >= kt) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int slot = tid + 256 * k;
      const int e = slot * VW;
      const int sl = e / hc, ho = e % hc;
      const bool ok = slot < nslot && s0 + sl < L;
#pragma unroll
      for (int i = 0; i < VW; ++i) {
        pk[k][i] = ok ? Pb[(ho + i) * L + s0 + sl] : 0.0;
        bt[k][i] = ok ? betab[(ho + i) * L + s0 + sl] : 0.0f;
      }
      cbi[k] = (int)(((h_lo + ho) / p.hpg - g_lo) * kT * kT) + sl;
    }
  }

  for (int64_t qt = q_first; qt < q_end; ++qt) {
    const int64_t t0 = qt * kT;
    const int64_t nrow = min((int64_t)kT, L - t0);
    if (qt < kt) {
      // above the diagonal: zeros
      for (int64_t r = 0; r < nrow; ++r) {
        float* orow = arow + ((t0 + r) * L + s0) * H;
        for (int slot = tid; slot < nslot; slot += 256) {
          const int e = slot * VW;
          const int sl = e / hc, ho = e % hc;
          if (s0 + sl >= L) continue;
          if (VW == 4) __builtin_nontemporal_store(f32x4v{0.f, 0.f, 0.f, 0.f}, (f32x4v*)(orow + sl * H + ho));
          else orow[sl * H + ho] = 0.f;
        }
      }
      continue;
    }
    __syncthreads();  // the previous tile's rows are written: sPq and sCB are free
    for (int e = tid; e < kT * hc; e += 256) {
      const int r = e % kT, hh = e / kT;
      sPq[r * HCp + hh] = r < nrow ? Pb[hh * L + t0 + r] : 0.0;
    }
    // C_t . B_s for the tile, per group of the chunk
    {
      const int tq = tid >> 3, sk = (tid & 7) * 4;
      for (int64_t gi = 0; gi < ngc; ++gi) {
        const int64_t g = g_lo + gi;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int64_t n0 = 0; n0 < N; n0 += kKC) {
          // stage C[t0 + r][g][n0 ..] and B[s0 + r][g][n0 ..] (B transposed)
#pragma unroll
          for (int rep = 0; rep < kKC / 32; ++rep) {
            const int r = tid >> 3, c = (tid & 7) * 4 + 32 * rep;
            const int64_t t = t0 + r, s = s0 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t n = n0 + c + i;
              sC[r * kCP + c + i] = (t < L && n < N) ? Act<T>::ld((const T*)a.C + ((b * L + t) * a.G + g) * N + n) : 0.f;
              sB[(c + i) * kT + r] = (s < L && n < N) ? Act<T>::ld((const T*)a.B + ((b * L + s) * a.G + g) * N + n) : 0.f;
            }
          }
          __syncthreads();
#pragma unroll 8
          for (int k = 0; k < kKC; ++k) {
            const float cv = sC[tq * kCP + k];
            const f32x4v bv = *(const f32x4v*)(sB + k * kT + sk);
            acc[0] = fmaf(cv, bv[0], acc[0]);
            acc[1] = fmaf(cv, bv[1], acc[1]);
            acc[2] = fmaf(cv, bv[2], acc[2]);
            acc[3] = fmaf(cv, bv[3], acc[3]);
          }
          __syncthreads();
        }
        *(f32x4v*)(sCB + (gi * kT + tq) * kT + sk) = f32x4v{acc[0], acc[1], acc[2], acc[3]};
      }
    }
    __syncthreads();
    // the rows: alpha[t][s0 + sl][h] = CB[t][s] * exp2(P[t] - P[s]) * betas_s for s <= t
    for (int64_t r = 0; r < nrow; ++r) {
      const int64_t t = t0 + r;
      float* orow = arow + (t * L + s0) * H;
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const int slot = tid + 256 * k;
        const int e = slot * VW;
        const int sl = e / hc, ho = e % hc;
        if (slot >= nslot || s0 + sl >= L) continue;
        float o[VW];
        if (s0 + sl > t) {
#pragma unroll
          for (int i = 0; i < VW; ++i) o[i] = 0.f;
        } else {
#pragma unroll
          for (int i = 0; i < VW; ++i) {
            const int gi_off = VW == 1 ? (int)(((h_lo + ho + i) / p.hpg - g_lo) * kT * kT) + sl : cbi[k];
            const float cb = sCB[gi_off + r * kT];
            const float e2 = (float)(sPq[r * HCp + ho + i] - pk[k][i]);
            o[i] = cb * fast_exp2(e2) * bt[k][i];
          }
        }
        if (VW == 4) __builtin_nontemporal_store(f32x4v{o[0], o[1 % VW], o[2 % VW], o[3 % VW]}, (f32x4v*)(orow + sl * H + ho));
        else orow[sl * H + ho] = o[0];
      }
    }
  }
}

AttnPlan make_plan(const AttnArgs& a) {
  AttnPlan p{};
  p.hpg = a.H / a.G;
  if (p.hpg <= kMaxHC) {
    int64_t gpc = kMaxHC / p.hpg;
    if (gpc > kMaxGPC) gpc = kMaxGPC;
    if (gpc > a.G) gpc = a.G;
    p.GPC = gpc;
    p.HC = gpc * p.hpg;
    p.cpg = 1;
    p.nchunks = (a.G + gpc - 1) / gpc;
  } else {
    p.GPC = 1;
    p.HC = kMaxHC;
    p.cpg = (p.hpg + kMaxHC - 1) / kMaxHC;
    p.nchunks = a.G * p.cpg;
  }
  p.nkt = (a.L + kT - 1) / kT;
  p.nqr = (p.nkt + kRange - 1) / kRange;
  return p;
}

size_t lds_bytes(const AttnPlan& p) {
  return (size_t)kT * p.HC * sizeof(double) + (size_t)p.GPC * kT * kT * sizeof(float) +
         (size_t)kT * kCP * sizeof(float) + (size_t)kKC * kT * sizeof(float);
}

// the largest plan: 128 heads and 8 groups per chunk
constexpr size_t lds_bytes_max() {
  return (size_t)kT * kMaxHC * sizeof(double) + (size_t)kMaxGPC * kT * kT * sizeof(float) +
         (size_t)kT * kCP * sizeof(float) + (size_t)kKC * kT * sizeof(float);
}

// Dynamic LDS beyond 64 KiB (up to 81 KiB here, of the 160 KiB a gfx950
// workgroup may hold) has to be allowed per kernel, once on each device.
template <typename T, int VW>
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, unsigned items, size_t lds, hipStream_t s) {
  static std::atomic<uint64_t> allowed{0};  // bit d: allowed on device d
  if (lds > 65536) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (!bit || !(allowed.load(std::memory_order_relaxed) & bit)) {
      e = hipFuncSetAttribute((const void*)ssd_attention_kernel<T, VW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_bytes_max());
      if (e != hipSuccess) return e;
      allowed.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  hipLaunchKernelGGL((ssd_attention_kernel<T, VW>), dim3(items), dim3(256), lds, s, a, p);
  return hipGetLastError();
}

}  // namespace

bool ssd_attention_supported(const AttnArgs& a) {
  if (a.G <= 0 || a.H % a.G != 0) return false;
  const AttnPlan p = make_plan(a);
  const double items = (double)a.batch * (double)p.nchunks * (double)p.nkt * (double)p.nqr;
  return items < 2147483647.0 && (double)a.batch * (double)a.H < 2147483647.0;
}

size_t ssd_attention_ws(const AttnArgs& a) {
  return (size_t)a.batch * (size_t)a.L * (size_t)a.H * (sizeof(double) + sizeof(float));
}

hipError_t launch_ssd_attention(const AttnArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  const AttnPlan p = make_plan(a);
  const unsigned items = (unsigned)(a.batch * p.nchunks * p.nkt * p.nqr);
  const size_t lds = lds_bytes(p);
  const bool vec = p.hpg % 4 == 0;
  const unsigned pblocks = (unsigned)(a.batch * a.H);
  if (a.bf16) {
    hipLaunchKernelGGL(attn_prefix_kernel<uint16_t>, dim3(pblocks), dim3(256), 0, s, a);
    return vec ? launch_attn<uint16_t, 4>(a, p, items, lds, s) : launch_attn<uint16_t, 1>(a, p, items, lds, s);
  }
  hipLaunchKernelGGL(attn_prefix_kernel<float>, dim3(pblocks), dim3(256), 0, s, a);
  return vec ? launch_attn<float, 4>(a, p, items, lds, s) : launch_attn<float, 1>(a, p, items, lds, s);
}

}  // namespace sscan
