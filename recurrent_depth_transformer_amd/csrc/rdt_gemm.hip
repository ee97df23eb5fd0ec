// MFMA GEMM kernels of the recurrent block (gfx950, wave64, bf16 or fp32 MFMA).
//
//   C = A . B^T with A [M, K] (rows optionally gathered through a token list)
//   and B [N, K] in the [out, in] layout of a linear layer, fp32 accumulation.
//
// One 256-thread workgroup computes a BM x BN tile; its four waves form a 2x2
// grid of (BM/2) x (BN/2) wave tiles built from 16x16x32 MFMAs. Each K stage
// moves 128 bytes per row (64 bf16 or 32 fp32) from HBM into registers while
// the previous stage is multiplied out of LDS. The fp32 tile then goes back
// through LDS so the epilogue can see whole head rows (RoPE pairs, SwiGLU gate
// and up halves, router rows) and write 16-byte coalesced vectors.
//
// Workgroups are renumbered so that consecutive logical tiles land on the same
// XCD (hardware places workgroup i on XCD i % 8), keeping tiles that share
// operands inside one L2.
#include "rdt_device.h"
#include "rdt_launch.h"

namespace rdt {

template <typename T, int BM, int BN>
struct GemmShape {
  static constexpr int BK = 128 / (int)sizeof(T);
  static constexpr int VEC = ST<T>::VEC;
  static constexpr int VPR = BK / VEC;  // 16-byte vectors per row per stage (8)
  static constexpr int LDK = BK + VEC;  // LDS row stride (elements), 16-byte pad
  static constexpr int A_LD = BM * VPR / 256;
  static constexpr int B_LD = BN * VPR / 256;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KSUB = BK / 32;
  static constexpr int CR = 64;         // epilogue rows per LDS chunk
  static constexpr int EPI_LD = BN + 4;
  static constexpr int SMEM_AB = (BM + BN) * LDK * (int)sizeof(T);
  static constexpr int SMEM_EPI = CR * EPI_LD * 4;
  static constexpr int SMEM = SMEM_AB > SMEM_EPI ? SMEM_AB : SMEM_EPI;
};

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int q = nb >> 3, rem = nb & 7;
  const int x = bid & 7, local = bid >> 3;
  return x * q + (x < rem ? x : rem) + local;
}

// Main loop: acc += A_rows . B_rows^T over K (and a second phase over K2).
template <typename T, int BM, int BN, bool TWO, typename S = GemmShape<T, BM, BN>>
__device__ __forceinline__ void gemm_mainloop(f32x4 (&acc)[S::FM][S::FN], char* smem,
                                              const T* (&ap)[S::A_LD], const T* (&bp)[S::B_LD], int K,
                                              const T* (&ap2)[S::A_LD], const T* (&bp2)[S::B_LD], int K2) {
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + BM * S::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kc = (tid % S::VPR) * S::VEC;
  const int nk1 = (K + S::BK - 1) / S::BK;
  const int nk = nk1 + (TWO ? (K2 + S::BK - 1) / S::BK : 0);

#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[S::A_LD], rb[S::B_LD];
  const uint4 zero = make_uint4(0, 0, 0, 0);
#define RDT_GLOAD(KT)                                                                  \
  {                                                                                    \
    const bool ph2 = TWO && (KT) >= nk1;                                               \
    const int k0 = (ph2 ? (KT)-nk1 : (KT)) * S::BK + kc;                               \
    const int Kp = ph2 ? K2 : K;                                                       \
    _Pragma("unroll") for (int i = 0; i < S::A_LD; ++i) {                              \
      const T* p = ph2 ? ap2[i] : ap[i];                                               \
      ra[i] = (p != nullptr && k0 < Kp) ? *reinterpret_cast<const uint4*>(p + k0) : make_uint4(0, 0, 0, 0); \
    }                                                                                  \
    _Pragma("unroll") for (int i = 0; i < S::B_LD; ++i) {                              \
      const T* p = ph2 ? bp2[i] : bp[i];                                               \
      rb[i] = (p != nullptr && k0 < Kp) ? *reinterpret_cast<const uint4*>(p + k0) : make_uint4(0, 0, 0, 0); \
    }                                                                                  \
  }
#define RDT_SSTORE()                                                                   \
  {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < S::A_LD; ++i) {                              \
      const int r = (tid + i * 256) / S::VPR;                                          \
      *reinterpret_cast<uint4*>(As + r * S::LDK + kc) = ra[i];                         \
    }                                                                                  \
    _Pragma("unroll") for (int i = 0; i < S::B_LD; ++i) {                              \
      const int r = (tid + i * 256) / S::VPR;                                          \
      *reinterpret_cast<uint4*>(Bs + r * S::LDK + kc) = rb[i];                         \
    }                                                                                  \
  }

  RDT_GLOAD(0)
  RDT_SSTORE()
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) RDT_GLOAD(kt + 1)
#pragma unroll
    for (int ks = 0; ks < S::KSUB; ++ks) {
      Frag<T> fa[S::FM], fb[S::FN];
      const int ko = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < S::FM; ++i)
        fa[i] = frag_lds<T>(As + (wm * S::WM + i * 16 + (lane & 15)) * S::LDK + ko);
#pragma unroll
      for (int j = 0; j < S::FN; ++j)
        fb[j] = frag_lds<T>(Bs + (wn * S::WN + j * 16 + (lane & 15)) * S::LDK + ko);
#pragma unroll
      for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      RDT_SSTORE()
      __syncthreads();
    }
  }
#undef RDT_GLOAD
#undef RDT_SSTORE
}

// Writes the accumulators of rows [c*CR, c*CR+CR) into the fp32 LDS tile.
template <typename T, int BM, int BN, typename S = GemmShape<T, BM, BN>>
__device__ __forceinline__ void acc_to_lds(const f32x4 (&acc)[S::FM][S::FN], float* Cs, int c) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if ((wm * S::WM) / S::CR != c) return;
  const int rb = wm * S::WM - c * S::CR;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(rb + i * 16 + (lane >> 4) * 4 + r) * S::EPI_LD + wn * S::WN + j * 16 + (lane & 15)] =
            acc[i][j][r];
}

// ============================================================== dense GEMM
template <typename T, int BM, int BN, bool TWO>
__global__ __launch_bounds__(256) void k_dense_gemm(DenseGemm g) {
  using S = GemmShape<T, BM, BN>;
  __shared__ __align__(16) char smem[S::SMEM];
  const int Mact = g.Mdev ? *g.Mdev : g.M;
  int ntot = 0;
  for (int s = 0; s < g.nseg; ++s) ntot += g.seg[s].ncols;
  const int ntn = (ntot + BN - 1) / BN;
  const int ntm = (g.M + BM - 1) / BM;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = L / ntm, mt = L % ntm;  // consecutive tiles share a B column block
  const int m0 = mt * BM, n0 = nt * BN;
  if (m0 >= Mact) return;
  const int z = blockIdx.z;
  const int tid = threadIdx.x;

  const T* ap[S::A_LD];
  const T* bp[S::B_LD];
  const T* ap2[S::A_LD];
  const T* bp2[S::B_LD];
  const T* A = reinterpret_cast<const T*>(g.A) + (long long)z * g.a_bstride;
#pragma unroll
  for (int i = 0; i < S::A_LD; ++i) {
    const int r = (tid + i * 256) / S::VPR;
    const int row = m0 + r;
    ap[i] = nullptr;
    ap2[i] = nullptr;
    if (row < Mact) {
      const int src = (g.gather && g.rows) ? g.rows[row] : row;
      ap[i] = A + (long long)src * g.lda;
      if (TWO) ap2[i] = reinterpret_cast<const T*>(g.A2) + (long long)row * g.lda2;
    }
  }
#pragma unroll
  for (int i = 0; i < S::B_LD; ++i) {
    const int c = n0 + (tid + i * 256) / S::VPR;
    bp[i] = nullptr;
    bp2[i] = nullptr;
    if (c < ntot) {
      int s = 0, base = 0;
      while (s + 1 < g.nseg && c >= base + g.seg[s].ncols) { base += g.seg[s].ncols; ++s; }
      bp[i] = reinterpret_cast<const T*>(g.seg[s].B) + (long long)z * g.b_bstride +
              (long long)(c - base) * g.K;
      if (TWO) bp2[i] = reinterpret_cast<const T*>(g.B2) + (long long)c * g.K2;
    }
  }

  f32x4 acc[S::FM][S::FN];
  gemm_mainloop<T, BM, BN, TWO>(acc, smem, ap, bp, g.K, ap2, bp2, g.K2);

  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int c = 0; c < BM / S::CR + (BM < S::CR ? 1 : 0); ++c) {
    acc_to_lds<T, BM, BN>(acc, Cs, c);
    __syncthreads();
    const int rbase = m0 + c * S::CR;
    const int nrows = BM < S::CR ? BM : S::CR;
    if (g.epi == EPI_STORE) {
      for (int idx = tid; idx < nrows * (BN / 8); idx += 256) {
        const int r = idx / (BN / 8), c8 = (idx % (BN / 8)) * 8;
        const int row = rbase + r, gc = n0 + c8;
        if (row >= Mact || gc >= ntot) continue;
        int s = 0, base = 0;
        while (s + 1 < g.nseg && gc >= base + g.seg[s].ncols) { base += g.seg[s].ncols; ++s; }
        const GemmSeg& sg = g.seg[s];
        const int lc = gc - base;
        const int tok = g.rows ? g.rows[row] : row;
        const int orow = sg.scatter ? tok : row;
        const float* crow = Cs + r * S::EPI_LD;
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x];
        if (sg.rope) {
          const int rd = g.rope_dim, half = rd >> 1;
          const int pos = tok % g.seq;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int hd = (lc + x) % rd;
            const int jj = hd % half;
            const float cs = g.cosb[pos * half + jj], sn = g.sinb[pos * half + jj];
            if (hd < half) {
              v[x] = crow[c8 + x] * cs - crow[c8 + x + half] * sn;
            } else {
              v[x] = crow[c8 + x - half] * sn + crow[c8 + x] * cs;
            }
          }
        }
        const long long off = (long long)z * g.c_bstride + (long long)orow * sg.ldc + lc;
        if (sg.out_f32) {
          store8<float>(reinterpret_cast<float*>(sg.C) + off, v);
        } else {
          store8<T>(reinterpret_cast<T*>(sg.C) + off, v);
        }
      }
    } else {  // EPI_ROUTER: one thread per row, E <= BN logits in the LDS row
      const RouterEpi& re = g.router;
      const int r = tid;
      const int row = rbase + r;
      if (r < nrows && row < Mact) {
        const float* crow = Cs + r * S::EPI_LD;
        const int E = re.E, k = re.k;
        float mx = -INFINITY;
        for (int e = 0; e < E; ++e) mx = fmaxf(mx, crow[e]);
        float den = 0.f;
        for (int e = 0; e < E; ++e) den += expf(crow[e] - mx);
        uint64_t taken = 0;
        float kth = 0.f;
        const int tok = g.rows ? g.rows[row] : row;
        for (int j = 0; j < k; ++j) {
          int bi = -1;
          float best = -INFINITY;
          for (int e = 0; e < E; ++e) {
            if ((taken >> e) & 1ull) continue;
            const float sv = crow[e] + (re.bias ? re.bias[e] : 0.f);
            if (bi < 0 || sv > best) { best = sv; bi = e; }
          }
          taken |= 1ull << bi;
          kth = best;
          re.idx[(long long)row * k + j] = bi;
          re.gates[(long long)row * k + j] = expf(crow[bi] - mx) / den;
          if (re.dump_idx) re.dump_idx[(long long)tok * k + j] = bi;
        }
        float gap = INFINITY;
        if (k < E) {
          float nxt = -INFINITY;
          int bi = -1;
          for (int e = 0; e < E; ++e) {
            if ((taken >> e) & 1ull) continue;
            const float sv = crow[e] + (re.bias ? re.bias[e] : 0.f);
            if (bi < 0 || sv > nxt) { nxt = sv; bi = e; }
          }
          gap = kth - nxt;
        }
        re.gap[row] = gap;
        if (re.dump_gap) re.dump_gap[tok] = gap;
      }
    }
    __syncthreads();
  }
}

template <typename T, int BM, int BN>
static hipError_t dense_launch(const DenseGemm& g, hipStream_t s) {
  int ntot = 0;
  for (int i = 0; i < g.nseg; ++i) ntot += g.seg[i].ncols;
  const int ntn = (ntot + BN - 1) / BN, ntm = (g.M + BM - 1) / BM;
  dim3 grid(ntn * ntm, 1, g.batch > 0 ? g.batch : 1);
  if (g.A2) {
    hipLaunchKernelGGL((k_dense_gemm<T, BM, BN, true>), grid, dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL((k_dense_gemm<T, BM, BN, false>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t dense_dispatch(const DenseGemm& g, hipStream_t s) {
  if (g.bm == 64 && g.bn == 64) return dense_launch<T, 64, 64>(g, s);
  if (g.bm == 64 && g.bn == 128) return dense_launch<T, 64, 128>(g, s);
  if (g.bm == 128 && g.bn == 64) return dense_launch<T, 128, 64>(g, s);
  return dense_launch<T, 128, 128>(g, s);
}

hipError_t launch_dense_gemm(const DenseGemm& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  return g.dtype == DT_F32 ? dense_dispatch<float>(g, s) : dense_dispatch<bf16_t>(g, s);
}

// ============================================================ grouped GEMM
template <typename T, int BM, int BN, int KIND>
__global__ __launch_bounds__(256) void k_grouped_gemm(GroupedGemm g) {
  using S = GemmShape<T, BM, BN>;
  __shared__ __align__(16) char smem[S::SMEM];
  const int G = g.E + g.Se;
  const int n = g.ndev ? *g.ndev : g.n_static;
  // KIND 0 produces BN/2 SwiGLU outputs per tile from BN/2 gate + BN/2 up rows
  const int OUTW = KIND == 0 ? BN / 2 : BN;
  const int ntn = (g.N + OUTW - 1) / OUTW;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = L / ntn, nt = L % ntn;  // consecutive tiles share the A rows
  const int total_mt = g.tile_start[G];
  if (mt >= total_mt) return;
  int grp = 0;
  while (grp + 1 < G && mt >= g.tile_start[grp + 1]) ++grp;
  const bool routed = grp < g.E;
  const int rows_g = routed ? g.counts[grp] : n;
  const int pbase = routed ? g.offs[grp] : n * g.k + (grp - g.E) * n;
  const int ml0 = (mt - g.tile_start[grp]) * BM;
  const int n0 = nt * OUTW;
  const int tid = threadIdx.x;
  const T* A = reinterpret_cast<const T*>(g.A);

  const T* ap[S::A_LD];
  const T* bp[S::B_LD];
#pragma unroll
  for (int i = 0; i < S::A_LD; ++i) {
    const int m = ml0 + (tid + i * 256) / S::VPR;
    ap[i] = nullptr;
    if (m < rows_g) {
      int src;
      if (KIND == 0) src = routed ? g.perm[pbase + m] : m;
      else src = pbase + m;
      ap[i] = A + (long long)src * g.lda;
    }
  }
  const long long wsz = (long long)g.N * g.K;  // one expert's matrix
  if (KIND == 0) {
    const T* wg = reinterpret_cast<const T*>(routed ? g.W1 : g.S1) + (routed ? grp : grp - g.E) * wsz;
    const T* wu = reinterpret_cast<const T*>(routed ? g.W2 : g.S2) + (routed ? grp : grp - g.E) * wsz;
#pragma unroll
    for (int i = 0; i < S::B_LD; ++i) {
      const int c = (tid + i * 256) / S::VPR;
      const int f = n0 + (c % (BN / 2));
      bp[i] = f < g.N ? ((c < BN / 2 ? wg : wu) + (long long)f * g.K) : nullptr;
    }
  } else {
    const T* wd = reinterpret_cast<const T*>(routed ? g.W1 : g.S1) + (routed ? grp : grp - g.E) * wsz;
#pragma unroll
    for (int i = 0; i < S::B_LD; ++i) {
      const int c = n0 + (tid + i * 256) / S::VPR;
      bp[i] = c < g.N ? wd + (long long)c * g.K : nullptr;
    }
  }

  f32x4 acc[S::FM][S::FN];
  gemm_mainloop<T, BM, BN, false>(acc, smem, ap, bp, g.K, ap, bp, 0);

  float* Cs = reinterpret_cast<float*>(smem);
  T* C = reinterpret_cast<T*>(g.C);
#pragma unroll 1
  for (int c = 0; c < BM / S::CR + (BM < S::CR ? 1 : 0); ++c) {
    acc_to_lds<T, BM, BN>(acc, Cs, c);
    __syncthreads();
    const int nrows = BM < S::CR ? BM : S::CR;
    for (int idx = tid; idx < nrows * (OUTW / 8); idx += 256) {
      const int r = idx / (OUTW / 8), c8 = (idx % (OUTW / 8)) * 8;
      const int m = ml0 + c * S::CR + r;
      const int col = n0 + c8;
      if (m >= rows_g || col >= g.N) continue;
      const float* crow = Cs + r * S::EPI_LD;
      float v[8];
      if (KIND == 0) {
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float gt = crow[c8 + x], up = crow[BN / 2 + c8 + x];
          v[x] = gt / (1.f + expf(-gt)) * up;
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x];
      }
      store8<T>(C + (long long)(pbase + m) * g.ldc + col, v);
    }
    __syncthreads();
  }
}

template <typename T>
static hipError_t grouped_dispatch(const GroupedGemm& g, hipStream_t s) {
  if (g.kind == 0) {
    const int ntn = (g.N + GU_BN / 2 - 1) / (GU_BN / 2);
    dim3 grid(g.max_mtiles * ntn);
    hipLaunchKernelGGL((k_grouped_gemm<T, GU_BM, GU_BN, 0>), grid, dim3(256), 0, s, g);
  } else {
    const int ntn = (g.N + DN_BN - 1) / DN_BN;
    dim3 grid(g.max_mtiles * ntn);
    hipLaunchKernelGGL((k_grouped_gemm<T, DN_BM, DN_BN, 1>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GroupedGemm& g, hipStream_t s) {
  if (g.max_mtiles <= 0) return hipSuccess;
  return g.dtype == DT_F32 ? grouped_dispatch<float>(g, s) : grouped_dispatch<bf16_t>(g, s);
}

}  // namespace rdt
