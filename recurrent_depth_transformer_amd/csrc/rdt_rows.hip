// Bandwidth-bound row kernels of the recurrent block: the two RMSNorms (the
// second fused with the router and the expert slot assignment), the MoE
// combine fused with the LTI injection, ACT halting and the active-list
// compaction, depth attention, and small utilities.
//
// Row kernels give one wave64 to one token row; each lane moves 16-byte
// vectors, so a row of D floats is read in D/256 fully coalesced passes.
#include "rdt_device.h"
#include "rdt_launch.h"

namespace rdt {

constexpr int MAXV = 16;  // float4 vectors per lane: rows up to 4096 wide

// ------------------------------------------------------------------ RMSNorm
// x = h[tok] + e[tok] (+ a[i]); out = x / sqrt(mean(x^2) + eps) * g
// angle table entry g of cos/sin (position g / (dr/2), frequency g % (dr/2)):
// the angle and its reduction to [-pi, pi] in double precision, the cosine and
// sine of the remainder in single precision
__device__ __forceinline__ void rope_entry(float* cosb, float* sinb, int dr, float base, int g) {
  const int half = dr >> 1;
  const int s = g / half, i = g % half;
  const double inv = exp2(-2.0 * (double)i / (double)dr * log2((double)base));
  const double ang = (double)s * inv;
  const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  float sn, cs;
  sincosf((float)r, &sn, &cs);
  cosb[g] = cs;
  sinb[g] = sn;
}

// NV = float4 vectors per lane that cover a row (D <= 256 * NV). Rows up to
// 1024 wide (NV <= 4) request all of their h, e and a vectors before using any
// (addresses clamped into the row, so no branch guards a load); wider rows
// take them a vector at a time. The sums are formed in the same order either way.
template <typename T, int NV>
__global__ __launch_bounds__(256) void k_norm(NormArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_blocks = (a.n + 3) / 4;
  if ((int)blockIdx.x >= row_blocks) {            // first-loop extras: RoPE tables
    int g = ((int)blockIdx.x - row_blocks) * 256 + threadIdx.x;
    for (int j = 0; j < 2; ++j) {
      if (!a.rope_cos[j]) continue;
      const int tot = a.rope_S[j] * (a.rope_dr[j] >> 1);
      if (g < tot) {
        rope_entry(a.rope_cos[j], a.rope_sin[j], a.rope_dr[j], a.rope_base, g);
        return;
      }
      g -= tot;
    }
    return;
  }
  if (blockIdx.x == 0 && a.zero)
    for (int z = threadIdx.x; z < a.zero_n; z += 256) a.zero[z] = 0;
  const int i = blockIdx.x * 4 + wave;
  const int n = a.ndev ? *a.ndev : a.n;
  if (i >= n) return;
  const int tok = a.rows ? a.rows[i] : i;
  const int D = a.D;
  float x[NV][4];
  float ss = 0.f;
  if constexpr (NV <= 4) {
    float4 hv[NV], ev[NV], av[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const int col = (c * 64 + lane) * 4;
      const int cc = col < D ? col : D - 4;
      hv[c] = *reinterpret_cast<const float4*>(a.h + (long long)tok * D + cc);
      ev[c] = *reinterpret_cast<const float4*>(a.e + (long long)tok * D + cc);
    }
    if (a.a) {
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const int col = (c * 64 + lane) * 4;
        av[c] = *reinterpret_cast<const float4*>(a.a + (long long)i * D + (col < D ? col : D - 4));
      }
    }
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const int col = (c * 64 + lane) * 4;
      if (col < D) {
        if (a.h_copy) *reinterpret_cast<float4*>(a.h_copy + (long long)tok * D + col) = hv[c];
        x[c][0] = hv[c].x + ev[c].x; x[c][1] = hv[c].y + ev[c].y; x[c][2] = hv[c].z + ev[c].z;
        x[c][3] = hv[c].w + ev[c].w;
        if (a.a) {
          x[c][0] += av[c].x; x[c][1] += av[c].y; x[c][2] += av[c].z; x[c][3] += av[c].w;
        }
        ss += x[c][0] * x[c][0] + x[c][1] * x[c][1] + x[c][2] * x[c][2] + x[c][3] * x[c][3];
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const int col = (c * 64 + lane) * 4;
      if (col < D) {
        const float4 hv = *reinterpret_cast<const float4*>(a.h + (long long)tok * D + col);
        if (a.h_copy) *reinterpret_cast<float4*>(a.h_copy + (long long)tok * D + col) = hv;
        const float4 ev = *reinterpret_cast<const float4*>(a.e + (long long)tok * D + col);
        x[c][0] = hv.x + ev.x; x[c][1] = hv.y + ev.y; x[c][2] = hv.z + ev.z; x[c][3] = hv.w + ev.w;
        if (a.a) {
          const float4 av = *reinterpret_cast<const float4*>(a.a + (long long)i * D + col);
          x[c][0] += av.x; x[c][1] += av.y; x[c][2] += av.z; x[c][3] += av.w;
        }
        ss += x[c][0] * x[c][0] + x[c][1] * x[c][1] + x[c][2] * x[c][2] + x[c][3] * x[c][3];
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
  T* out = reinterpret_cast<T*>(a.out) + (long long)(a.out_scatter ? tok : i) * D;
  T* dump = a.dump ? reinterpret_cast<T*>(a.dump) + (long long)tok * D : nullptr;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int col = (c * 64 + lane) * 4;
    if (col < D) {
      const float4 gv = *reinterpret_cast<const float4*>(a.g + col);
      float y[4] = {x[c][0] * inv * gv.x, x[c][1] * inv * gv.y, x[c][2] * inv * gv.z,
                    x[c][3] * inv * gv.w};
      store4<T>(out + col, y);
      if (dump) store4<T>(dump + col, y);
    }
  }
}

template <typename T>
static void norm_nv(const NormArgs& a, dim3 grid, hipStream_t s) {
  if (a.D <= 256) hipLaunchKernelGGL((k_norm<T, 1>), grid, dim3(256), 0, s, a);
  else if (a.D <= 512) hipLaunchKernelGGL((k_norm<T, 2>), grid, dim3(256), 0, s, a);
  else if (a.D <= 1024) hipLaunchKernelGGL((k_norm<T, 4>), grid, dim3(256), 0, s, a);
  else if (a.D <= 2048) hipLaunchKernelGGL((k_norm<T, 8>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_norm<T, MAXV>), grid, dim3(256), 0, s, a);
}

hipError_t launch_norm(const NormArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  long long extra = 0;
  for (int j = 0; j < 2; ++j)
    if (a.rope_cos[j]) extra += (long long)a.rope_S[j] * (a.rope_dr[j] / 2);
  dim3 grid((unsigned)((a.n + 3) / 4 + (extra + 255) / 256));
  if (a.D > 256 * MAXV) return hipErrorInvalidValue;
  if (a.dtype == DT_F32) norm_nv<float>(a, grid, s);
  else norm_nv<bf16_t>(a, grid, s);
  return hipGetLastError();
}

// ---------------------------------------------------- ACT active-list compaction
// Runs at the end of every combine workgroup, inside the combine launch. Each
// workgroup holds 4 consecutive rows of the input list (in token order) and
// knows which of them keep running (halting sum still below the threshold).
// It publishes that 4-bit mask with an arrival bit through a device-coherent
// store, then counts itself on `done`; the workgroup that counts last (no
// workgroup ever waits for another before that) builds the stable compacted
// list: an exclusive scan of the masks, then every kept token in order, the
// per-sequence offsets, and it clears the masks and the counter for the next
// launch. A mask whose store is not yet visible to it is re-read (its store
// was issued before its workgroup counted itself, so it arrives; the re-read
// is bounded all the same). Only workgroups holding rows count themselves,
// on CMP_SUB sub-counters and one counter of finished sub-counters, because
// atomics on one address serialise (one counter for 4096 workgroups cost
// about 75 us per launch).
constexpr int CMP_ARRIVED = 0x100;

constexpr int CMP_SUB = 64;   // arrival sub-counters (same-address atomics serialise)

__device__ __forceinline__ void act_compact_tail(const CombineArgs& a, int n, int keep_bits) {
  constexpr int SC = __HIP_MEMORY_SCOPE_AGENT;
  __shared__ int s_last;
  __shared__ int s_ws[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwg = (n + 3) / 4;     // workgroups holding rows of the list
  const int w = blockIdx.x;
  if (nwg == 0) {                  // nothing ran: an empty list
    if (w == 0) {
      if (tid == 0) *a.n_out = 0;
      for (int b = tid; b <= a.nseq; b += 256) a.seg_out[b] = 0;
    }
    return;
  }
  if (w >= nwg) return;
  // done[0] counts finished sub-counters, done[1 + j] the workgroups w with
  // w % CMP_SUB == j; the one completing the last sub-counter goes on
  if (tid == 0) {
    __hip_atomic_store(a.wg_mask + w, keep_bits | CMP_ARRIVED, __ATOMIC_RELAXED, SC);
    asm volatile("" ::: "memory");
    const int j = w % CMP_SUB;
    const int tgt = (nwg - 1 - j) / CMP_SUB + 1;
    int last = 0;
    if (__hip_atomic_fetch_add(a.done + 1 + j, 1, __ATOMIC_RELAXED, SC) == tgt - 1) {
      __hip_atomic_store(a.done + 1 + j, 0, __ATOMIC_RELAXED, SC);          // zero for the next launch
      const int nsub = nwg < CMP_SUB ? nwg : CMP_SUB;
      last = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, SC) == nsub - 1;
    }
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  // the last workgroup: thread tid takes the input workgroups [w0, w1)
  const int chunk = (nwg + 255) / 256;
  const int w0 = tid * chunk < nwg ? tid * chunk : nwg;
  const int w1 = w0 + chunk < nwg ? w0 + chunk : nwg;
  int cntl = 0;
  for (int b0 = w0; b0 < w1; b0 += 16) {
    int mm[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      mm[u] = b0 + u < w1 ? __hip_atomic_load(a.wg_mask + b0 + u, __ATOMIC_RELAXED, SC) : CMP_ARRIVED;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (b0 + u >= w1) break;
      int m = mm[u];
      for (int spin = 0; !(m & CMP_ARRIVED) && spin < (1 << 20); ++spin) {
        __builtin_amdgcn_s_sleep(2);
        m = __hip_atomic_load(a.wg_mask + b0 + u, __ATOMIC_RELAXED, SC);
      }
      a.wg_tmp[b0 + u] = m & 15;
      cntl += __popc(m & 15);
      __hip_atomic_store(a.wg_mask + b0 + u, 0, __ATOMIC_RELAXED, SC);   // zero for the next launch
    }
  }
  // exclusive scan of the per-thread counts over the workgroup
  int inc = cntl;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) s_ws[wave] = inc;
  __syncthreads();
  int run = inc - cntl;
  for (int q = 0; q < wave; ++q) run += s_ws[q];
  const int total = s_ws[0] + s_ws[1] + s_ws[2] + s_ws[3];
  for (int w = w0; w < w1; ++w) {
    const int m = a.wg_tmp[w];
    a.wg_tmp[w] = (run << 4) | m;             // base of input workgroup w, and its mask
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if ((m >> r) & 1) a.rows_out[run++] = a.rows ? a.rows[4 * w + r] : 4 * w + r;
  }
  if (tid == 0) {
    *a.n_out = total;
    __hip_atomic_store(a.done, 0, __ATOMIC_RELAXED, SC);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // seg_out[b]: kept rows before input position seg_in[b]
  for (int b = tid; b <= a.nseq; b += 256) {
    const int j = a.seg_in[b];
    int v = total;
    if (j < n) {
      const int x = a.wg_tmp[j >> 2];
      v = (x >> 4) + __popc((x & 15) & ((1 << (j & 3)) - 1));
    }
    a.seg_out[b] = v;
  }
}

// ---------------------------------------------------------- combine + inject
template <typename T, int NV, bool LAT>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr bool PRE = LAT && NV <= 4;  // h, e, a ahead of the scan (registers)
  constexpr int KP = LAT ? 8 : 0;       // routing entries fetched ahead
  constexpr int KA = KP > 0 ? KP : 1;
  __shared__ int s_off[MAX_EXPERTS];
  __shared__ int s_keep;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int n = a.ndev ? *a.ndev : a.n;
  if (blockIdx.x > 0 && (int)blockIdx.x * 4 >= n) return;   // as in k_combine8
  const bool live = i < n;
  const int D = a.D, k = a.k;
  if (threadIdx.x == 0) s_keep = 0;
  int colc[NV];
  bool okc[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int col = (c * 64 + lane) * 4;
    okc[c] = col < D;
    colc[c] = okc[c] ? col : 0;
  }
  const int tok = live ? (a.rows ? a.rows[i] : i) : 0;
  int eidx[KA], eslot[KA];
  float egt[KA];
  float4 hv[NV], ev[NV], av[NV];
#pragma unroll
  for (int j = 0; j < KA; ++j) { eidx[j] = 0; eslot[j] = 0; egt[j] = 0.f; }
  if (live) {
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (j < k) {
        eidx[j] = a.idx[(long long)i * k + j];
        eslot[j] = a.slot[(long long)i * k + j];
        egt[j] = a.gates[(long long)i * k + j];
      }
    if constexpr (PRE) {
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        hv[c] = *reinterpret_cast<const float4*>(a.h + (long long)tok * D + colc[c]);
        ev[c] = *reinterpret_cast<const float4*>(a.e + (long long)tok * D + colc[c]);
        av[c] = *reinterpret_cast<const float4*>(a.a + (long long)i * D + colc[c]);
      }
    }
  }
  // exclusive prefix of the per-expert counts (wave 0, one lane per expert)
  if (wave == 0) {
    const int c = lane < a.E ? a.cnt[lane] : 0;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < a.E) s_off[lane] = inc - c;
    if (blockIdx.x == 0 && lane < a.E) {
      if (a.counts_dump) a.counts_dump[lane] = c;
      a.cnt_next[lane] = 0;                        // the next loop's router starts from zero
    }
  }
  __syncthreads();
  if (live) {
  const T* Y = reinterpret_cast<const T*>(a.Y);
  // expert output row p, columns col..col+3: stored values, or the sum of the
  // K-slice partials in slice order
  auto yrow = [&](long long p, int col, float* y) {
    if (a.ksplit > 1) {
      const float4 v0 = *reinterpret_cast<const float4*>(a.Yp + p * D + col);
      y[0] = v0.x; y[1] = v0.y; y[2] = v0.z; y[3] = v0.w;
      for (int s = 1; s < a.ksplit; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(a.Yp + s * a.ystride + p * D + col);
        y[0] += v.x; y[1] += v.y; y[2] += v.z; y[3] += v.w;
      }
    } else {
      load4f<T>(Y + p * D + col, y);
    }
  };
  float m[NV][4];
#pragma unroll
  for (int c = 0; c < NV; ++c) m[c][0] = m[c][1] = m[c][2] = m[c][3] = 0.f;
  // routed experts in pairs (the second of a pair may repeat the first row
  // and is then not added); each element adds its experts in choice order
#pragma unroll
  for (int j0 = 0; j0 < KP; j0 += 2) {
    if (j0 >= k) break;
    const bool two = j0 + 1 < k;
    const long long p0 = s_off[eidx[j0]] + eslot[j0];
    const long long p1 = two ? s_off[eidx[j0 + 1]] + eslot[j0 + 1] : p0;
    float y0[NV][4], y1[NV][4];
    if (a.ksplit == 2) {
      float4 u0[NV], u1[NV], w0[NV], w1[NV];
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        u0[c] = *reinterpret_cast<const float4*>(a.Yp + p0 * D + colc[c]);
        u1[c] = *reinterpret_cast<const float4*>(a.Yp + a.ystride + p0 * D + colc[c]);
        w0[c] = *reinterpret_cast<const float4*>(a.Yp + p1 * D + colc[c]);
        w1[c] = *reinterpret_cast<const float4*>(a.Yp + a.ystride + p1 * D + colc[c]);
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        y0[c][0] = u0[c].x + u1[c].x; y0[c][1] = u0[c].y + u1[c].y;
        y0[c][2] = u0[c].z + u1[c].z; y0[c][3] = u0[c].w + u1[c].w;
        y1[c][0] = w0[c].x + w1[c].x; y1[c][1] = w0[c].y + w1[c].y;
        y1[c][2] = w0[c].z + w1[c].z; y1[c][3] = w0[c].w + w1[c].w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        yrow(p0, colc[c], y0[c]);
        yrow(p1, colc[c], y1[c]);
      }
    }
    const float g0 = egt[j0], g1 = egt[j0 + 1 < KA ? j0 + 1 : j0];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      m[c][0] += g0 * y0[c][0]; m[c][1] += g0 * y0[c][1]; m[c][2] += g0 * y0[c][2]; m[c][3] += g0 * y0[c][3];
      if (two) {
        m[c][0] += g1 * y1[c][0]; m[c][1] += g1 * y1[c][1]; m[c][2] += g1 * y1[c][2]; m[c][3] += g1 * y1[c][3];
      }
    }
  }
  // (outside LAT, loads stay behind per-column guards: fewer registers live)
  for (int j = KP; j < k; ++j) {
    const long long p = s_off[a.idx[(long long)i * k + j]] + a.slot[(long long)i * k + j];
    const float gt = a.gates[(long long)i * k + j];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      if (LAT || okc[c]) {
        float y[4];
        yrow(p, colc[c], y);
        m[c][0] += gt * y[0]; m[c][1] += gt * y[1]; m[c][2] += gt * y[2]; m[c][3] += gt * y[3];
      }
    }
  }
  const float sw = a.smax ? a.smax[i] : 1.f;   // shared-expert weight
  for (int s = 0; s < a.Se; ++s) {
    const long long p = (long long)n * k + (long long)s * n + i;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      if (LAT || okc[c]) {
        float y[4];
        yrow(p, colc[c], y);
        m[c][0] += sw * y[0]; m[c][1] += sw * y[1]; m[c][2] += sw * y[2]; m[c][3] += sw * y[3];
      }
    }
  }
  float z = 0.f, ss = 0.f;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    if (!okc[c]) continue;
    const int col = colc[c];
    if constexpr (!PRE) {
      hv[c] = *reinterpret_cast<const float4*>(a.h + (long long)tok * D + col);
      ev[c] = *reinterpret_cast<const float4*>(a.e + (long long)tok * D + col);
      av[c] = *reinterpret_cast<const float4*>(a.a + (long long)i * D + col);
    }
    if (a.d) {
      const float4 dv = *reinterpret_cast<const float4*>(a.d + (long long)i * D + col);
      m[c][0] += dv.x; m[c][1] += dv.y; m[c][2] += dv.z; m[c][3] += dv.w;
    }
    const float4 Av = *reinterpret_cast<const float4*>(a.A + col);
    const float4 Bv = *reinterpret_cast<const float4*>(a.B + col);
    float4 hn;
    hn.x = Av.x * hv[c].x + Bv.x * ev[c].x + av[c].x + m[c][0];
    hn.y = Av.y * hv[c].y + Bv.y * ev[c].y + av[c].y + m[c][1];
    hn.z = Av.z * hv[c].z + Bv.z * ev[c].z + av[c].z + m[c][2];
    hn.w = Av.w * hv[c].w + Bv.w * ev[c].w + av[c].w + m[c][3];
    *reinterpret_cast<float4*>(a.h + (long long)tok * D + col) = hn;
    if (a.a_dump) *reinterpret_cast<float4*>(a.a_dump + (long long)tok * D + col) = av[c];
    if (a.act) {
      const float4 wv = *reinterpret_cast<const float4*>(a.w_halt + col);
      z += wv.x * hn.x + wv.y * hn.y + wv.z * hn.z + wv.w * hn.w;
    }
    // u = h' + e for the next loop's first RMSNorm
    m[c][0] = hn.x + ev[c].x; m[c][1] = hn.y + ev[c].y; m[c][2] = hn.z + ev[c].z; m[c][3] = hn.w + ev[c].w;
    ss += m[c][0] * m[c][0] + m[c][1] * m[c][1] + m[c][2] * m[c][2] + m[c][3] * m[c][3];
  }
  if (a.n1_out) {
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
    T* dst = reinterpret_cast<T*>(a.n1_out) + (long long)tok * D;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      if (!okc[c]) continue;
      const int col = colc[c];
      const float4 gv = *reinterpret_cast<const float4*>(a.g1 + col);
      float y[4] = {m[c][0] * inv * gv.x, m[c][1] * inv * gv.y, m[c][2] * inv * gv.z, m[c][3] * inv * gv.w};
      store4<T>(dst + col, y);
    }
  }
  if (a.act) {
    z = wave_sum(z);
    if (lane == 0) {
      const float p = 1.f / (1.f + expf(-z));
      const float c = a.cum[tok] + p;
      a.cum[tok] = c;
      if (a.cum_dump) a.cum_dump[tok] = c;
      if (c < a.thr) atomicOr(&s_keep, 1 << wave);
    }
  }
  if (lane == 0 && a.loops) a.loops[tok] = a.t + 1;
  }  // live
  if (a.act && a.rows_out) {
    __syncthreads();
    act_compact_tail(a, n, s_keep);
  }
}

// The combine with 8 consecutive columns per lane (bf16 expert outputs as one
// 16-byte load, float rows as two): the bandwidth form for rows that are a
// multiple of 512 wide. Expert outputs are gathered EB rows at a time (all
// their loads in flight). Every element adds the same terms in the same order
// as k_combine; the per-lane partial sums of the halting dot product and of
// the next RMSNorm run over the lane's own columns.
template <int NV8, int EB>
__global__ __launch_bounds__(256) void k_combine8(CombineArgs a) {
  __shared__ int s_off[MAX_EXPERTS];
  __shared__ int s_keep;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int n = a.ndev ? *a.ndev : a.n;
  // the grid covers the static row count: past the running rows only
  // workgroup 0 has work (clearing the next loop's counts); the ACT
  // compaction involves only the workgroups that hold rows
  if (blockIdx.x > 0 && (int)blockIdx.x * 4 >= n) return;
  const bool live = i < n;
  const int D = a.D, k = a.k;
  if (threadIdx.x == 0) s_keep = 0;
  if (wave == 0) {   // exclusive prefix of the per-expert counts
    const int c = lane < a.E ? a.cnt[lane] : 0;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < a.E) s_off[lane] = inc - c;
    if (blockIdx.x == 0 && lane < a.E) {
      if (a.counts_dump) a.counts_dump[lane] = c;
      a.cnt_next[lane] = 0;
    }
  }
  __syncthreads();
  if (live) {
    const int tok = a.rows ? a.rows[i] : i;
    const bf16_t* Y = reinterpret_cast<const bf16_t*>(a.Y);
    float m[NV8][8];
#pragma unroll
    for (int c = 0; c < NV8; ++c)
#pragma unroll
      for (int x = 0; x < 8; ++x) m[c][x] = 0.f;
    const float sw = a.smax ? a.smax[i] : 1.f;   // shared-expert weight
    const int KT = k + a.Se;                     // routed choices in order, then the shared experts
    for (int j0 = 0; j0 < KT; j0 += EB) {
      long long p[EB];
      float gt[EB];
#pragma unroll
      for (int u = 0; u < EB; ++u) {
        const int j = j0 + u < KT ? j0 + u : j0;
        if (j < k) {
          p[u] = s_off[a.idx[(long long)i * k + j]] + a.slot[(long long)i * k + j];
          gt[u] = a.gates[(long long)i * k + j];
        } else {
          p[u] = (long long)n * k + (long long)(j - k) * n + i;
          gt[u] = sw;
        }
      }
      uint4 yv[EB][NV8];
#pragma unroll
      for (int u = 0; u < EB; ++u)
#pragma unroll
        for (int c = 0; c < NV8; ++c)
          yv[u][c] = *reinterpret_cast<const uint4*>(Y + p[u] * D + (c * 64 + lane) * 8);
#pragma unroll
      for (int u = 0; u < EB; ++u) {
        if (j0 + u >= KT) break;
#pragma unroll
        for (int c = 0; c < NV8; ++c) {
          const uint32_t w4[4] = {yv[u][c].x, yv[u][c].y, yv[u][c].z, yv[u][c].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            m[c][2 * q] += gt[u] * __uint_as_float(w4[q] << 16);
            m[c][2 * q + 1] += gt[u] * __uint_as_float(w4[q] & 0xffff0000u);
          }
        }
      }
    }
    float z = 0.f, ss = 0.f;
#pragma unroll
    for (int c = 0; c < NV8; ++c) {
      const int col0 = (c * 64 + lane) * 8;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = col0 + 4 * hh;
        float* mm = m[c] + 4 * hh;
        const float4 hv = *reinterpret_cast<const float4*>(a.h + (long long)tok * D + col);
        const float4 ev = *reinterpret_cast<const float4*>(a.e + (long long)tok * D + col);
        const float4 av = *reinterpret_cast<const float4*>(a.a + (long long)i * D + col);
        if (a.d) {
          const float4 dv = *reinterpret_cast<const float4*>(a.d + (long long)i * D + col);
          mm[0] += dv.x; mm[1] += dv.y; mm[2] += dv.z; mm[3] += dv.w;
        }
        const float4 Av = *reinterpret_cast<const float4*>(a.A + col);
        const float4 Bv = *reinterpret_cast<const float4*>(a.B + col);
        float4 hn;
        hn.x = Av.x * hv.x + Bv.x * ev.x + av.x + mm[0];
        hn.y = Av.y * hv.y + Bv.y * ev.y + av.y + mm[1];
        hn.z = Av.z * hv.z + Bv.z * ev.z + av.z + mm[2];
        hn.w = Av.w * hv.w + Bv.w * ev.w + av.w + mm[3];
        *reinterpret_cast<float4*>(a.h + (long long)tok * D + col) = hn;
        if (a.a_dump) *reinterpret_cast<float4*>(a.a_dump + (long long)tok * D + col) = av;
        if (a.act) {
          const float4 wv = *reinterpret_cast<const float4*>(a.w_halt + col);
          z += wv.x * hn.x + wv.y * hn.y + wv.z * hn.z + wv.w * hn.w;
        }
        mm[0] = hn.x + ev.x; mm[1] = hn.y + ev.y; mm[2] = hn.z + ev.z; mm[3] = hn.w + ev.w;
        ss += mm[0] * mm[0] + mm[1] * mm[1] + mm[2] * mm[2] + mm[3] * mm[3];
      }
    }
    if (a.n1_out) {
      ss = wave_sum(ss);
      const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
      bf16_t* dst = reinterpret_cast<bf16_t*>(a.n1_out) + (long long)tok * D;
#pragma unroll
      for (int c = 0; c < NV8; ++c) {
        const int col = (c * 64 + lane) * 8;
        const float4 g0 = *reinterpret_cast<const float4*>(a.g1 + col);
        const float4 g1 = *reinterpret_cast<const float4*>(a.g1 + col + 4);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float y[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) y[x] = m[c][x] * inv * gg[x];
        store8<bf16_t>(dst + col, y);
      }
    }
    if (a.act) {
      z = wave_sum(z);
      if (lane == 0) {
        const float p = 1.f / (1.f + expf(-z));
        const float c = a.cum[tok] + p;
        a.cum[tok] = c;
        if (a.cum_dump) a.cum_dump[tok] = c;
        if (c < a.thr) atomicOr(&s_keep, 1 << wave);
      }
    }
    if (lane == 0 && a.loops) a.loops[tok] = a.t + 1;
  }
  if (a.act && a.rows_out) {
    __syncthreads();
    act_compact_tail(a, n, s_keep);
  }
}

template <typename T, bool LAT>
static hipError_t combine_nv(const CombineArgs& a, hipStream_t s) {
  dim3 grid((a.n + 3) / 4);
  const int nv = (a.D + 255) / 256;
  if (nv <= 1) hipLaunchKernelGGL((k_combine<T, 1, LAT>), grid, dim3(256), 0, s, a);
  else if (nv <= 2) hipLaunchKernelGGL((k_combine<T, 2, LAT>), grid, dim3(256), 0, s, a);
  else if (nv <= 4) hipLaunchKernelGGL((k_combine<T, 4, LAT>), grid, dim3(256), 0, s, a);
  else if (nv <= 8) hipLaunchKernelGGL((k_combine<T, 8, LAT>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_combine<T, 16, LAT>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t combine_t(const CombineArgs& a, hipStream_t s) {
  // up to 2048 rows (512 workgroups, one round on the chip at LAT's occupancy)
  if (a.n <= 2048) return combine_nv<T, true>(a, s);
  // long bf16 launches with whole 512-column vectors per row: 8 columns per
  // lane (measured on 8192 rows of 2048: 153 -> 137 us)
  if (sizeof(T) == 2 && a.ksplit <= 1 && a.D % 512 == 0 && a.D <= 4096) {
    const dim3 grid((a.n + 3) / 4);
    switch (a.D / 512) {
      case 1: hipLaunchKernelGGL((k_combine8<1, 5>), grid, dim3(256), 0, s, a); return hipGetLastError();
      case 2: hipLaunchKernelGGL((k_combine8<2, 5>), grid, dim3(256), 0, s, a); return hipGetLastError();
      case 4: hipLaunchKernelGGL((k_combine8<4, 5>), grid, dim3(256), 0, s, a); return hipGetLastError();
      case 8: hipLaunchKernelGGL((k_combine8<8, 3>), grid, dim3(256), 0, s, a); return hipGetLastError();
      default: break;
    }
  }
  return combine_nv<T, false>(a, s);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  return a.dtype == DT_F32 ? combine_t<float>(a, s) : combine_t<bf16_t>(a, s);
}


// ----------------------------------------- second RMSNorm + router + slots
// A workgroup of 16 waves takes 16 compacted rows. Each wave forms one row
// x = h + e + a, n2 = RMSNorm(x) * g2 (stored in the storage type, and staged
// in LDS in column chunks). The router logits n2 . Wr^T of the 16 rows come
// from 16x16x32 MFMAs: wave w takes expert tile (w % NT) and every (16/NT)-th
// k-step, partial tiles are summed through LDS. Then one wave per row: softmax
// gates over all experts, top-k on logit + bias by k rounds of a wave argmax
// (equal scores go to the lower expert). Expert slots: the workgroup counts
// its picks per expert in LDS, reserves a contiguous range of slots per
// expert with one atomic add on cnt, and hands the slots out; the slot order
// inside an expert is arbitrary (each row's expert output does not depend on
// which rows share its GEMM tile).
// Up to 2048-wide rows the kernel is held to 64 VGPRs (8 waves per SIMD), so
// two 16-wave workgroups share a CU and all of a 8192-row launch is resident
// at once (measured on 8192 x 2048: 75 -> 67 us).
// LAT (launches of up to a few thousand rows, one round of at most 256
// workgroups): the kernel may use 128 VGPRs, and every term of a row and the
// router weights of four k-steps are requested before any is used; the sums
// are formed in the same order as in the bandwidth form, so both forms give
// identical results.
template <typename T, int NV, bool LAT>
__global__ __launch_bounds__(1024, (NV <= 8 && !LAT) ? 8 : 1) void k_norm_route(NormRouteArgs a) {
  constexpr int KC = 4096 / (int)sizeof(T);        // columns per LDS chunk
  constexpr int LDA = KC + 16 / (int)sizeof(T);    // padded row stride
  __shared__ __align__(16) T As[16 * LDA];
  __shared__ int s_idx[16][MAX_EXPERTS];         // chosen experts of the 16 rows
  __shared__ int s_cnt[MAX_EXPERTS], s_base[MAX_EXPERTS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const NormArgs& na = a.norm;
  const int i = blockIdx.x * 16 + wave;
  const int n = na.ndev ? *na.ndev : na.n;
  // the grid covers the static row count; under ACT fewer rows run, and a
  // workgroup without any has nothing to do (uniform across the workgroup,
  // before any barrier)
  if ((int)blockIdx.x * 16 >= n) return;
  const int D = na.D, E = a.E, k = a.k;
  const bool live = i < n;
  const int tok = live ? (na.rows ? na.rows[i] : i) : 0;
  float x[NV][4];
  float ss = 0.f;
  if constexpr (LAT) {
#pragma unroll
    for (int c = 0; c < NV; ++c) x[c][0] = x[c][1] = x[c][2] = x[c][3] = 0.f;
    if (live) {   // one row per wave (NV may exceed the row's chunks: every column is checked)
      float4 t[4][NV];
      const float* src[4] = {na.h + (long long)tok * D, na.e + (long long)tok * D,
                             na.a2 ? na.a2 + (long long)i * D : nullptr, na.a ? na.a + (long long)i * D : nullptr};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          const int col = (c * 64 + lane) * 4;
          t[q][c] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (src[q] && col < D) t[q][c] = *reinterpret_cast<const float4*>(src[q] + col);
        }
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        // (h + e) + depth-attention output + attention output, as below
        x[c][0] = t[0][c].x + t[1][c].x; x[c][1] = t[0][c].y + t[1][c].y;
        x[c][2] = t[0][c].z + t[1][c].z; x[c][3] = t[0][c].w + t[1][c].w;
#pragma unroll
        for (int q = 2; q < 4; ++q)
          if (src[q]) { x[c][0] += t[q][c].x; x[c][1] += t[q][c].y; x[c][2] += t[q][c].z; x[c][3] += t[q][c].w; }
        ss += x[c][0] * x[c][0] + x[c][1] * x[c][1] + x[c][2] * x[c][2] + x[c][3] * x[c][3];
      }
    }
  } else
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int col = (c * 64 + lane) * 4;
    x[c][0] = x[c][1] = x[c][2] = x[c][3] = 0.f;
    if (live && col < D) {
      const float4 hv = *reinterpret_cast<const float4*>(na.h + (long long)tok * D + col);
      const float4 ev = *reinterpret_cast<const float4*>(na.e + (long long)tok * D + col);
      x[c][0] = hv.x + ev.x; x[c][1] = hv.y + ev.y; x[c][2] = hv.z + ev.z; x[c][3] = hv.w + ev.w;
      if (na.a2) {  // depth-attention output (Dreamer sequential block)
        const float4 dv = *reinterpret_cast<const float4*>(na.a2 + (long long)i * D + col);
        x[c][0] += dv.x; x[c][1] += dv.y; x[c][2] += dv.z; x[c][3] += dv.w;
      }
      if (na.a) {   // attention output (absent in the parallel block)
        const float4 av = *reinterpret_cast<const float4*>(na.a + (long long)i * D + col);
        x[c][0] += av.x; x[c][1] += av.y; x[c][2] += av.z; x[c][3] += av.w;
      }
      ss += x[c][0] * x[c][0] + x[c][1] * x[c][1] + x[c][2] * x[c][2] + x[c][3] * x[c][3];
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)D + na.eps);
  T* out = reinterpret_cast<T*>(na.out) + (long long)i * D;
  T* dump = na.dump && live ? reinterpret_cast<T*>(na.dump) + (long long)tok * D : nullptr;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int col = (c * 64 + lane) * 4;
    if (live && col < D) {
      const float4 gv = *reinterpret_cast<const float4*>(na.g + col);
      x[c][0] *= inv * gv.x; x[c][1] *= inv * gv.y; x[c][2] *= inv * gv.z; x[c][3] *= inv * gv.w;
      store4<T>(out + col, x[c]);
      if (dump) store4<T>(dump + col, x[c]);
    }
  }
  // router logits on the stored (rounded) values
  const int NT = E <= 16 ? 1 : E <= 32 ? 2 : 4;   // expert tiles of 16
  const int KS = 16 / NT;                          // waves sharing one expert tile
  const int nt = wave % NT, ks = wave / NT;
  const int en = nt * 16 + (lane & 15);            // expert of this lane's B row
  const T* Wr = reinterpret_cast<const T*>(a.Wr);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kc0 = 0; kc0 < D; kc0 += KC) {
    const int ck = D - kc0 < KC ? D - kc0 : KC;
    const int ck32 = (ck + 31) & ~31;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const int col = (c * 64 + lane) * 4;        // global column
      const int lc = col - kc0;                   // column inside the chunk
      if (lc >= 0 && lc < ck32) store4<T>(As + wave * LDA + lc, x[c]);   // zero beyond D
    }
    __syncthreads();
    const int nstep = ck32 / 32;
    if constexpr (LAT) {
      // this wave's k-steps ks, ks + KS, ... four at a time: the weight
      // fragments are fetched together (addresses clamped into the matrix,
      // values zeroed where the expert or column does not exist), then
      // multiplied in k-step order
      const int my = nstep > ks ? (nstep - ks + KS - 1) / KS : 0;
      const T* wrow = Wr + (long long)(en < E ? en : 0) * D;
      for (int b0 = 0; b0 < my; b0 += 4) {
        Frag<T> af[4], bf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kk = (ks + (b0 + u) * KS) * 32 + (lane >> 4) * 8;
          const bool ok = en < E && b0 + u < my && kc0 + kk < D;
          const uint4* q = reinterpret_cast<const uint4*>(wrow + (ok ? kc0 + kk : 0));
#pragma unroll
          for (int v = 0; v < (int)(sizeof(T) / 2); ++v) {
            const uint4 w = q[v];
            bf[u].v[v] = ok ? w : make_uint4(0, 0, 0, 0);
          }
          af[u] = frag_lds<T>(As + (lane & 15) * LDA + (b0 + u < my ? kk : 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (b0 + u < my) mma(acc, af[u], bf[u]);
      }
    } else
    for (int st = ks; st < nstep; st += KS) {
      const int kk = st * 32 + (lane >> 4) * 8;
      const Frag<T> af = frag_lds<T>(As + (lane & 15) * LDA + kk);
      Frag<T> bf = frag_zero<T>();
      if (en < E && kc0 + kk < D) {
        const uint4* q = reinterpret_cast<const uint4*>(Wr + (long long)en * D + kc0 + kk);
#pragma unroll
        for (int v = 0; v < (int)(sizeof(T) / 2); ++v) bf.v[v] = q[v];
      }
      mma(acc, af, bf);
    }
    __syncthreads();
  }
  // partial tiles -> LDS (reusing the staging buffer), summed per row below
  float* red = reinterpret_cast<float*>(As);      // [KS][16][64]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(ks * 16 + (lane >> 4) * 4 + r) * 64 + nt * 16 + (lane & 15)] = acc[r];
  __syncthreads();
  if (live) {
    const bool own = lane < E;                     // lane e holds expert e
    float logit = 0.f;
    for (int q = 0; q < KS; ++q) logit += red[(q * 16 + wave) * 64 + lane];
    const float mx = wave_max(own ? logit : -INFINITY);
    const float pe = own ? expf(logit - mx) : 0.f;
    const float den = wave_sum(pe);
    const float gate = pe / den;
    if (lane == 0 && a.smax) a.smax[i] = 1.f / den;  // the largest probability: exp(0) / den
    float sel = own ? logit + (a.bias ? a.bias[lane] : 0.f) : -INFINITY;
    bool avail = own;                              // not chosen yet
    float kth = 0.f;
    for (int j = 0; j < k; ++j) {
      const float best = wave_max(avail ? sel : -INFINITY);
      unsigned long long m = __ballot(avail && sel == best);
      if (m == 0ull) m = __ballot(avail);          // NaN scores: first free expert (k <= E)
      const int win = __ffsll((long long)m) - 1;   // lowest expert among equal scores
      const float g = __shfl(gate, win, 64);
      if (lane == 0) {
        s_idx[wave][j] = win;
        a.gates[(long long)i * k + j] = g;
        if (a.dump_idx) a.dump_idx[(long long)tok * k + j] = win;
      }
      if (lane == win) avail = false;
      kth = best;
    }
    const float nxt = wave_max(avail ? sel : -INFINITY);
    if (lane == 0) {
      const float gp = k < E ? kth - nxt : INFINITY;
      a.gap[i] = gp;
      if (a.dump_gap) a.dump_gap[tok] = gp;
    }
  }
  // expert slots: local ranks through LDS counters, one global reservation
  // per expert and workgroup
  if (threadIdx.x < MAX_EXPERTS) s_cnt[threadIdx.x] = 0;
  __syncthreads();
  int local = 0, ex = -1;
  const int q = threadIdx.x;                       // pick q = (row r, choice j)
  const int r = q / (k > 0 ? k : 1), jj = q - r * k;
  const int row = blockIdx.x * 16 + r;
  if (q < 16 * k && row < n) {
    ex = s_idx[r][jj];
    local = atomicAdd(&s_cnt[ex], 1);
  }
  __syncthreads();
  if ((int)threadIdx.x < E && s_cnt[threadIdx.x] > 0) s_base[threadIdx.x] = atomicAdd(&a.cnt[threadIdx.x], s_cnt[threadIdx.x]);
  __syncthreads();
  if (ex >= 0) {
    const int sl = s_base[ex] + local;
    a.idx[(long long)row * k + jj] = ex;
    a.slot[(long long)row * k + jj] = sl;
    a.pcap[(long long)ex * a.cap + sl] = row;
  }
}

template <typename T>
static hipError_t norm_route_t(const NormRouteArgs& a, hipStream_t s) {
  dim3 grid((a.norm.n + 15) / 16);
  const int nv = (a.norm.D + 255) / 256;
  // up to 4096 rows of up to 1024 columns: at most 256 workgroups, one per CU,
  // so the latency form's registers cost no occupancy that matters (wider
  // rows would spill its four terms of NV vectors)
  if (a.norm.n <= 4096 && nv <= 4) {
    if (nv <= 1) hipLaunchKernelGGL((k_norm_route<T, 1, true>), grid, dim3(1024), 0, s, a);
    else if (nv <= 2) hipLaunchKernelGGL((k_norm_route<T, 2, true>), grid, dim3(1024), 0, s, a);
    else hipLaunchKernelGGL((k_norm_route<T, 4, true>), grid, dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  if (nv <= 1) hipLaunchKernelGGL((k_norm_route<T, 1, false>), grid, dim3(1024), 0, s, a);
  else if (nv <= 2) hipLaunchKernelGGL((k_norm_route<T, 2, false>), grid, dim3(1024), 0, s, a);
  else if (nv <= 4) hipLaunchKernelGGL((k_norm_route<T, 4, false>), grid, dim3(1024), 0, s, a);
  else if (nv <= 8) hipLaunchKernelGGL((k_norm_route<T, 8, false>), grid, dim3(1024), 0, s, a);
  else hipLaunchKernelGGL((k_norm_route<T, 16, false>), grid, dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_route(const NormRouteArgs& a, hipStream_t s) {
  if (a.norm.n <= 0 || a.E > MAX_EXPERTS || a.E < 1 || a.k > a.E || a.norm.D % 8 || 16 * a.k > 1024)
    return hipErrorInvalidValue;
  return a.norm.dtype == DT_F32 ? norm_route_t<float>(a, s) : norm_route_t<bf16_t>(a, s);
}


// ----------------------------------------------------------- MLA latents
// cqn = RMSNorm(c_q) * gq;  latent = [RMSNorm(c_kv) * gkv | rope(k_rope)]
template <typename T>
__global__ __launch_bounds__(256) void k_mla_norm(MlaNormArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int n = a.ndev ? *a.ndev : a.n;
  if (i >= n) return;
  const int tok = a.rows ? a.rows[i] : i;
  // c_q
  {
    const float* src = a.cq_raw + (long long)tok * a.ql;
    float ss = 0.f;
    for (int c = lane; c < a.ql; c += 64) ss += src[c] * src[c];
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)a.ql + a.eps);
    T* dst = reinterpret_cast<T*>(a.cqn) + (long long)tok * a.ql;
    for (int c = lane; c < a.ql; c += 64) dst[c] = ST<T>::from_f(src[c] * inv * a.gq[c]);
  }
  const int W = a.kvl + a.nr;
  const float* src = a.lat_raw + (long long)tok * W;
  T* dst = reinterpret_cast<T*>(a.latent) + (long long)tok * W;
  {
    float ss = 0.f;
    for (int c = lane; c < a.kvl; c += 64) ss += src[c] * src[c];
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)a.kvl + a.eps);
    for (int c = lane; c < a.kvl; c += 64) dst[c] = ST<T>::from_f(src[c] * inv * a.gkv[c]);
  }
  const int half = a.nr >> 1;
  const int pos = a.pos_dev ? *a.pos_dev : tok % a.S;
  for (int j = lane; j < half; j += 64) {
    const float x1 = src[a.kvl + j], x2 = src[a.kvl + j + half];
    const float cs = a.cosb[pos * half + j], sn = a.sinb[pos * half + j];
    dst[a.kvl + j] = ST<T>::from_f(x1 * cs - x2 * sn);
    dst[a.kvl + j + half] = ST<T>::from_f(x1 * sn + x2 * cs);
  }
}

// The same arithmetic with every value a row needs requested before any is
// used (c_q up to 64 * NQ columns, the latent of kvl <= 128 columns, its
// 32-wide rope part and the RoPE factors), so a wave waits on one round trip
// rather than one per pass.
template <typename T, int NQ>
__global__ __launch_bounds__(256) void k_mla_norm_batched(MlaNormArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int n = a.ndev ? *a.ndev : a.n;
  if (i >= n) return;
  const int tok = a.rows ? a.rows[i] : i;
  const int W = a.kvl + a.nr, half = a.nr >> 1;
  const float* cs = a.cq_raw + (long long)tok * a.ql;
  const float* src = a.lat_raw + (long long)tok * W;
  const int pos = a.pos_dev ? *a.pos_dev : tok % a.S;
  float cq[NQ], gqv[NQ], lk[2], gk[2];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int c = lane + 64 * u;
    cq[u] = c < a.ql ? cs[c] : 0.f;
    gqv[u] = c < a.ql ? a.gq[c] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    lk[u] = c < a.kvl ? src[c] : 0.f;
    gk[u] = c < a.kvl ? a.gkv[c] : 0.f;
  }
  const bool rj = lane < half;
  const int j = rj ? lane : 0;
  const float x1 = src[a.kvl + j], x2 = src[a.kvl + j + half];
  const float co = a.cosb[pos * half + j], sn = a.sinb[pos * half + j];
  {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NQ; ++u) ss += cq[u] * cq[u];
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)a.ql + a.eps);
    T* dst = reinterpret_cast<T*>(a.cqn) + (long long)tok * a.ql;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = lane + 64 * u;
      if (c < a.ql) dst[c] = ST<T>::from_f(cq[u] * inv * gqv[u]);
    }
  }
  T* dst = reinterpret_cast<T*>(a.latent) + (long long)tok * W;
  {
    float ss = lk[0] * lk[0];
    ss += lk[1] * lk[1];
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)a.kvl + a.eps);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = lane + 64 * u;
      if (c < a.kvl) dst[c] = ST<T>::from_f(lk[u] * inv * gk[u]);
    }
  }
  if (rj) {
    dst[a.kvl + j] = ST<T>::from_f(x1 * co - x2 * sn);
    dst[a.kvl + j + half] = ST<T>::from_f(x1 * sn + x2 * co);
  }
}

hipError_t launch_mla_norm(const MlaNormArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((a.n + 3) / 4);
  const int nq = (a.ql + 63) / 64;
  if (a.kvl <= 128 && a.nr <= 128 && nq <= 8) {
#define RDT_MN(Q)                                                                                  \
    if (nq <= Q) {                                                                                 \
      if (a.dtype == DT_F32) hipLaunchKernelGGL((k_mla_norm_batched<float, Q>), grid, dim3(256), 0, s, a); \
      else hipLaunchKernelGGL((k_mla_norm_batched<bf16_t, Q>), grid, dim3(256), 0, s, a);          \
      return hipGetLastError();                                                                    \
    }
    RDT_MN(2) RDT_MN(4) RDT_MN(6) RDT_MN(8)
#undef RDT_MN
  }
  if (a.dtype == DT_F32) hipLaunchKernelGGL(k_mla_norm<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_mla_norm<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// rope of the per-head query rope slice into the attention query buffer
template <typename T>
__global__ __launch_bounds__(256) void k_qrope(QRopeArgs a) {
  const int half = a.nr >> 1;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int n = a.ndev ? *a.ndev : a.n;
  const long long per_row = (long long)a.H * half;
  const int i = (int)(gid / per_row);
  if (i >= n) return;
  const int rem = (int)(gid % per_row);
  const int h = rem / half, j = rem % half;
  const int tok = a.rows ? a.rows[i] : i;
  const int pos = a.pos_dev ? *a.pos_dev : tok % a.S;
  const T* s = reinterpret_cast<const T*>(a.src) + (long long)i * a.src_ld + (long long)h * a.src_hs + a.src_off;
  T* d = reinterpret_cast<T*>(a.dst) + (long long)i * a.dst_ld + (long long)h * a.dst_hs + a.dst_off;
  const float x1 = ST<T>::to_f(s[j]), x2 = ST<T>::to_f(s[j + half]);
  const float cs = a.cosb[pos * half + j], sn = a.sinb[pos * half + j];
  d[j] = ST<T>::from_f(x1 * cs - x2 * sn);
  d[j + half] = ST<T>::from_f(x1 * sn + x2 * cs);
}

// bf16, 32-wide rope slices at 16-byte aligned offsets: one thread per (row,
// head) moves the slice and its RoPE factors as 16-byte vectors; the same
// arithmetic per element as k_qrope
__global__ __launch_bounds__(256) void k_qrope_vec(QRopeArgs a) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int n = a.ndev ? *a.ndev : a.n;
  const int i = (int)(gid / a.H), h = (int)(gid % a.H);
  if (i >= n) return;
  const int tok = a.rows ? a.rows[i] : i;
  const int pos = a.pos_dev ? *a.pos_dev : tok % a.S;
  const uint4* s = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.src) + (long long)i * a.src_ld +
                                                  (long long)h * a.src_hs + a.src_off);
  uint4* d = reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(a.dst) + (long long)i * a.dst_ld +
                                      (long long)h * a.dst_hs + a.dst_off);
  const float4* cb = reinterpret_cast<const float4*>(a.cosb + pos * 16);
  const float4* sb = reinterpret_cast<const float4*>(a.sinb + pos * 16);
  uint4 xr[4];
  float4 cr[4], sr[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { xr[v] = s[v]; cr[v] = cb[v]; sr[v] = sb[v]; }
  const bf16_t* x = reinterpret_cast<const bf16_t*>(xr);
  const float* co = reinterpret_cast<const float*>(cr);
  const float* sn = reinterpret_cast<const float*>(sr);
  bf16_t y[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float x1 = bf2f(x[j]), x2 = bf2f(x[j + 16]);
    y[j] = f2bf(x1 * co[j] - x2 * sn[j]);
    y[j + 16] = f2bf(x1 * sn[j] + x2 * co[j]);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) d[v] = reinterpret_cast<const uint4*>(y)[v];
}

hipError_t launch_qrope(const QRopeArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.dtype == DT_BF16 && a.nr == 32 && a.src_ld % 8 == 0 && a.src_hs % 8 == 0 && a.src_off % 8 == 0 &&
      a.dst_ld % 8 == 0 && a.dst_hs % 8 == 0 && a.dst_off % 8 == 0) {
    const long long tot = (long long)a.n * a.H;
    hipLaunchKernelGGL(k_qrope_vec, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const long long tot = (long long)a.n * a.H * (a.nr / 2);
  dim3 grid((unsigned)((tot + 255) / 256));
  if (a.dtype == DT_F32) hipLaunchKernelGGL(k_qrope<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_qrope<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------------------------- utilities
// RoPE angles in double precision: angle(s, i) = s * base^(-2i/dr)
__global__ void k_rope_tables(float* cosb, float* sinb, int S, int dr, float base) {
  const int half = dr >> 1;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= S * half) return;
  const int s = gid / half, i = gid % half;
  const double inv = pow((double)base, -2.0 * (double)i / (double)dr);
  const double ang = (double)s * inv;
  cosb[gid] = (float)cos(ang);
  sinb[gid] = (float)sin(ang);
}

hipError_t launch_rope_tables(float* cosb, float* sinb, int S, int dr, float base, hipStream_t s) {
  const int tot = S * (dr / 2);
  hipLaunchKernelGGL(k_rope_tables, dim3((tot + 255) / 256), dim3(256), 0, s, cosb, sinb, S, dr, base);
  return hipGetLastError();
}

template <typename V>
__global__ void k_fill(V* p, V v, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

static unsigned fill_blocks(long long n) {
  long long b = (n + 255) / 256;
  return (unsigned)(b < 4096 ? (b < 1 ? 1 : b) : 4096);
}

hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill<int>, dim3(fill_blocks(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill<float>, dim3(fill_blocks(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t launch_fill_u16(uint16_t* p, uint16_t v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill<uint16_t>, dim3(fill_blocks(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

__global__ void k_iota(int* p, int n, int* count, int count_val, int* seg, int B, int S) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid < n) p[gid] = gid;
  if (gid == 0 && count) *count = count_val;
  if (seg && gid <= B) seg[gid] = gid * S;
}

hipError_t launch_iota(int* p, int n, int* count, int count_val, int* seg, int B, int S, hipStream_t s) {
  const int tot = n > B + 1 ? n : B + 1;
  hipLaunchKernelGGL(k_iota, dim3((tot + 255) / 256), dim3(256), 0, s, p, n, count, count_val, seg, B, S);
  return hipGetLastError();
}

__global__ void k_copy_f32(float4* dst, const float4* src, long long n4) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy_f32(float* dst, const float* src, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long n4 = n / 4;  // callers pass multiples of 4
  hipLaunchKernelGGL(k_copy_f32, dim3(fill_blocks(n4)), dim3(256), 0, s, reinterpret_cast<float4*>(dst),
                     reinterpret_cast<const float4*>(src), n4);
  return hipGetLastError();
}

// --------------------------------------------------------- depth attention
// A wave serves one token and 256/dd of its query heads: a head owns dd/4
// consecutive lanes, each holding 4 of its elements, so the dot products
// reduce over dd/4 lanes only. Keys and values of loops 0..t of the same
// token; online softmax in loop order.
template <typename T>
__global__ __launch_bounds__(256) void k_depth_attention(DepthAttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dd = a.dd, lph = dd >> 2, hpw = 64 / lph;   // lanes per head, heads per wave
  const int wpt = (a.H + hpw - 1) / hpw;                 // waves per token
  const long long job = (long long)blockIdx.x * 4 + wave;
  if (job >= (long long)a.n * wpt) return;
  const int i = (int)(job / wpt);
  const int h = (int)(job % wpt) * hpw + lane / lph;
  const bool on = h < a.H;
  const int e0 = (lane % lph) * 4;
  const int kvh = on ? (h * a.KV) / a.H : 0;
  const long long kvoff = (long long)i * a.KV * dd + (long long)kvh * dd + e0;
  float q[4] = {0.f, 0.f, 0.f, 0.f}, o[4] = {0.f, 0.f, 0.f, 0.f};
  if (on) load4f<T>(reinterpret_cast<const T*>(a.q) + (long long)i * a.H * dd + (long long)h * dd + e0, q);
  float mrun = -INFINITY, lrun = 0.f;
  const float sc2 = a.scale * 1.4426950408889634f;   // scale * log2(e)
  // the keys and values of CH loops are requested before any is used (loop
  // indices past t repeat loop t: valid addresses, no branch around the
  // loads), then taken in loop order
  constexpr int CH = 8;
  for (int tau0 = 0; tau0 <= a.t; tau0 += CH) {
    float k[CH][4], v[CH][4];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int tau = tau0 + u <= a.t ? tau0 + u : a.t;
      const long long off = (long long)tau * a.lstride + (on ? kvoff : 0);
      load4f<T>(reinterpret_cast<const T*>(a.k) + off, k[u]);
      load4f<T>(reinterpret_cast<const T*>(a.v) + off, v[u]);
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (tau0 + u > a.t) break;
      float kk[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (on) {
#pragma unroll
        for (int x = 0; x < 4; ++x) { kk[x] = k[u][x]; vv[x] = v[u][x]; }
      }
      float s = q[0] * kk[0] + q[1] * kk[1] + q[2] * kk[2] + q[3] * kk[3];
      for (int off = lph >> 1; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      s *= sc2;   // scores in the base-2 domain: softmax is unchanged
      const float mnew = fmaxf(mrun, s);
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew), p = __builtin_amdgcn_exp2f(s - mnew);
      lrun = lrun * alpha + p;
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = o[x] * alpha + p * vv[x];
      mrun = mnew;
    }
  }
  if (on) {
    const float inv = 1.f / lrun;
    float r[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    store4<T>(reinterpret_cast<T*>(a.o) + (long long)i * a.H * dd + (long long)h * dd + e0, r);
  }
}

hipError_t launch_depth_attention(const DepthAttnArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.dd < 16 || a.dd > 128 || (a.dd & (a.dd - 1)) || a.t < 0 || a.H % a.KV) return hipErrorInvalidValue;
  const int hpw = 256 / a.dd;
  const long long jobs = (long long)a.n * ((a.H + hpw - 1) / hpw);
  dim3 grid((unsigned)((jobs + 3) / 4));
  if (a.dtype == DT_F32) hipLaunchKernelGGL(k_depth_attention<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_depth_attention<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------- router-bias balancing update
// One workgroup per bias row r. c_e = tokens expert e received in the loops
// that select with row r (loop t uses row min(t, rows - 1)); every expert
// below the row's mean load gains gamma, every expert above it loses gamma.
// The comparison is exact: total vs E * c_e in 64-bit integers.
__global__ __launch_bounds__(256) void k_bias_update(const int* counts, int T, int E, float* bias, int rows,
                                                     float gamma) {
  __shared__ long long part[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  auto load = [&](int e) {
    long long c = 0;
    for (int t = 0; t < T; ++t)
      if ((t < rows - 1 ? t : rows - 1) == r) c += counts[(long long)t * E + e];
    return c;
  };
  long long acc = 0;
  for (int e = tid; e < E; e += 256) acc += load(e);
  part[tid] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) part[tid] += part[tid + o];
    __syncthreads();
  }
  const long long total = part[0];
  for (int e = tid; e < E; e += 256) {
    const long long d = total - (long long)E * load(e);
    const float sg = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    bias[(long long)r * E + e] += gamma * sg;
  }
}

hipError_t launch_bias_update(const int* counts, int T, int E, float* bias, int rows, float gamma, hipStream_t s) {
  if (rows <= 0 || E <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bias_update, dim3(rows), dim3(256), 0, s, counts, T, E, bias, rows, gamma);
  return hipGetLastError();
}

// ---------------------------------------------------- expert depth usage
__global__ __launch_bounds__(256) void k_expert_depths(const int* counts, int T, int E, int* depths) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int d = 0;
  for (int t = 0; t < T; ++t) d += counts[(long long)t * E + e] > 0;
  depths[e] = d;
}

hipError_t launch_expert_depths(const int* counts, int T, int E, int* depths, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_expert_depths, dim3((E + 255) / 256), dim3(256), 0, s, counts, T, E, depths);
  return hipGetLastError();
}

// ------------------------------------------------------------ row scatter
__global__ __launch_bounds__(256) void k_rows_scatter(char* dst, long long dst_ld, const char* src, long long src_ld,
                                                      int vecs, int nrows, int s_in, int s_out, const int* pos_dev) {
  const int pos0 = pos_dev ? *pos_dev : 0;
  const long long n = (long long)nrows * vecs;
  for (long long x = blockIdx.x * 256ll + threadIdx.x; x < n; x += (long long)gridDim.x * 256) {
    const int r = (int)(x / vecs), v = (int)(x % vecs);
    const long long dr = (long long)(r / s_in) * s_out + r % s_in + pos0;
    *reinterpret_cast<uint4*>(dst + dr * dst_ld + v * 16) =
        *reinterpret_cast<const uint4*>(src + (long long)r * src_ld + v * 16);
  }
}

hipError_t launch_rows_scatter(void* dst, long long dst_ld, const void* src, long long src_ld, int bytes, int nrows,
                               int s_in, int s_out, const int* pos_dev, hipStream_t s) {
  if (nrows <= 0) return hipSuccess;
  if (bytes % 16 || s_in <= 0) return hipErrorInvalidValue;
  const int vecs = bytes / 16;
  const long long n = (long long)nrows * vecs;
  const int blocks = (int)(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(k_rows_scatter, dim3(blocks), dim3(256), 0, s, (char*)dst, dst_ld, (const char*)src, src_ld,
                     vecs, nrows, s_in, s_out, pos_dev);
  return hipGetLastError();
}

template <typename T>
__global__ void k_head_transpose(T* dst, const T* src, int H, int rows, int cols) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long tot = (long long)H * rows * cols;
  if (gid >= tot) return;
  const int i = (int)(gid % rows);
  const long long r = gid / rows;
  const int c = (int)(r % cols);
  const int h = (int)(r / cols);
  dst[gid] = src[((long long)h * rows + i) * cols + c];
}

hipError_t launch_head_transpose(int dtype, void* dst, const void* src, int H, int rows, int cols,
                                 hipStream_t s) {
  const long long tot = (long long)H * rows * cols;
  dim3 grid((unsigned)((tot + 255) / 256));
  if (dtype == DT_F32)
    hipLaunchKernelGGL(k_head_transpose<float>, grid, dim3(256), 0, s, (float*)dst, (const float*)src, H, rows, cols);
  else
    hipLaunchKernelGGL(k_head_transpose<bf16_t>, grid, dim3(256), 0, s, (bf16_t*)dst, (const bf16_t*)src, H, rows,
                       cols);
  return hipGetLastError();
}

}  // namespace rdt
