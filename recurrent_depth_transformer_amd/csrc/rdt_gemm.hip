// MFMA GEMM kernels of the recurrent block (gfx950, wave64, bf16 or fp32 MFMA).
//
//   C = A . B^T with A [M, K] (rows optionally gathered through a token list)
//   and B [N, K] in the [out, in] layout of a linear layer, fp32 accumulation.
//
// One workgroup computes a BM x BN tile; its NW waves (4 or 8) form an
// (NW/2) x 2 grid of (BM/(NW/2)) x (BN/2) wave tiles built from 16x16x32
// MFMAs. Each K stage
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

template <typename T, int BM, int BN, int NW = 4>
struct GemmShape {
  static constexpr int NT = NW * 64;    // threads per workgroup
  static constexpr int BK = 128 / (int)sizeof(T);
  static constexpr int VEC = ST<T>::VEC;
  static constexpr int VPR = BK / VEC;  // 16-byte vectors per row per stage (8)
  static constexpr int LDK = BK + VEC;  // LDS row stride (elements), 16-byte pad
  static constexpr int A_LD = BM * VPR / NT;
  static constexpr int B_LD = BN * VPR / NT;
  static constexpr int WM = BM / (NW / 2), WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KSUB = BK / 32;
  static constexpr int CR = 32;         // epilogue rows per LDS chunk
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

// ---------------------------------------------------------------------------
// bf16 main loop: an NS-stage ring of direct global->LDS loads.
//
// Each stage holds 64 k-values (128 bytes) of BM A-rows and BN B-rows. A wave
// load instruction moves 64 lanes x 16 bytes into 1 KB of LDS in lane order
// (8 rows x 128 bytes), so the row layout cannot be padded; instead lane l of a
// row r fetches the 16-byte k-chunk (l % 8) ^ (r % 8), which makes the 16-row
// fragment reads of the MFMA operands conflict-free. Loads for stage kt+NS-1
// are issued while stage kt is multiplied, one barrier per stage. Lanes whose
// row has no data load a valid dummy row (their products only reach discarded
// outputs); k-chunks past the end of K are zeroed in LDS after they land.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, int NW = 4>
struct LdsRing {
  static constexpr int RR = NW * 8;                 // rows per load round (16 bytes per lane)
  static constexpr int RB = NW * 1024;              // bytes per load round
  static constexpr int AL = BM / RR, BL = BN / RR;  // load rounds per stage
  static constexpr int LPS = AL + BL;               // load instructions per thread per stage
  static constexpr int STAGE = (BM + BN) * 128;     // bytes per stage (>= the fp32 epilogue chunk)
  static constexpr int WM = BM / (NW / 2);          // wave tile rows
  static constexpr int FM = WM / 16, FN = BN / 32;  // 16x16 fragments per wave
};

// Waits until at most n vector-memory operations of this wave are in flight.
// Written as asm with a memory clobber so that no LDS access moves across it.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define RDT_W(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    RDT_W(1) RDT_W(2) RDT_W(3) RDT_W(4) RDT_W(5) RDT_W(6) RDT_W(8) RDT_W(10) RDT_W(12) RDT_W(16) RDT_W(20) RDT_W(24)
#undef RDT_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// One wave-wide direct load: every lane moves 16 bytes from src into LDS at
// lds + 16 * lane. Issued through asm so that the compiler does not insert
// conservative waits for the LDS write; the ring waits explicitly (wait_vmcnt).
// m0 (the LDS base of the load) is set inside the same asm statement; the
// compiler keeps nothing of its own in m0 in these kernels (the generated code
// has no other m0 access), so the clobber cannot disturb it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

typedef __attribute__((address_space(3))) char lds_char;

// Stage buffers are distinct __shared__ objects and the loop is unrolled by NS,
// so every LDS access names its stage statically: the compiler can then tell the
// DMA writes of one stage from the reads of another and does not serialise them.
template <int BM, int BN, int NS, bool TWO, int NW, typename R = LdsRing<BM, BN, NS, NW>>
__device__ __forceinline__ void gemm_mainloop_ring(f32x4 (&acc)[R::FM][R::FN], char* const (&L)[NS],
                                                   const bf16_t* (&ap)[R::AL], const bf16_t* (&bp)[R::BL],
                                                   int K, const bf16_t* (&ap2)[R::AL],
                                                   const bf16_t* (&bp2)[R::BL], int K2, const bf16_t* adummy,
                                                   const bf16_t* bdummy, const bf16_t* adummy2,
                                                   const bf16_t* bdummy2) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int prow = tid >> 3;                        // row within a load round
  const int kchunk = ((tid & 7) ^ ((prow >> 1) & 7)) * 8;  // logical k offset this lane loads
  const int nk1 = (K + 63) >> 6;
  const int nk = nk1 + (TWO ? (K2 + 63) >> 6 : 0);

#pragma unroll
  for (int i = 0; i < R::FM; ++i)
#pragma unroll
    for (int j = 0; j < R::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int kt, char* buf) {
    const bool ph2 = TWO && kt >= nk1;
    const int k = (ph2 ? kt - nk1 : kt) * 64 + kchunk;
    const int Kp = ph2 ? K2 : K;
    const uint32_t st = (uint32_t)(uintptr_t)(lds_char*)buf + __builtin_amdgcn_readfirstlane(wave) * 1024;
#pragma unroll
    for (int i = 0; i < R::AL; ++i) {
      const bf16_t* p = ph2 ? ap2[i] : ap[i];
      const bf16_t* src = (p != nullptr && k < Kp) ? p + k : (ph2 ? adummy2 : adummy);
      dma16(src, st + i * R::RB);
    }
#pragma unroll
    for (int i = 0; i < R::BL; ++i) {
      const bf16_t* p = ph2 ? bp2[i] : bp[i];
      const bf16_t* src = (p != nullptr && k < Kp) ? p + k : (ph2 ? bdummy2 : bdummy);
      dma16(src, st + BM * 128 + i * R::RB);
    }
  };
  // one of the LPS load instructions of a stage (idx < AL: A rows, else B rows)
  auto issue_one = [&](int kt, char* buf, int idx) {
    const bool ph2 = TWO && kt >= nk1;
    const int k = (ph2 ? kt - nk1 : kt) * 64 + kchunk;
    const int Kp = ph2 ? K2 : K;
    const uint32_t st = (uint32_t)(uintptr_t)(lds_char*)buf + __builtin_amdgcn_readfirstlane(wave) * 1024;
    if (idx < R::AL) {
      const bf16_t* p = ph2 ? ap2[idx] : ap[idx];
      dma16((p != nullptr && k < Kp) ? p + k : (ph2 ? adummy2 : adummy), st + idx * R::RB);
    } else {
      const bf16_t* p = ph2 ? bp2[idx - R::AL] : bp[idx - R::AL];
      dma16((p != nullptr && k < Kp) ? p + k : (ph2 ? bdummy2 : bdummy), st + BM * 128 + (idx - R::AL) * R::RB);
    }
  };
  // zero this lane's k-chunks that lie past the end of K (after they landed)
  auto zero_tail = [&](int kt, char* buf) {
    const bool ph2 = TWO && kt >= nk1;
    const int k = (ph2 ? kt - nk1 : kt) * 64 + kchunk;
    const int Kp = ph2 ? K2 : K;
    if (k < Kp) return;
    char* st = buf + tid * 16;
#pragma unroll
    for (int i = 0; i < R::AL; ++i) *reinterpret_cast<uint4*>(st + i * R::RB) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < R::BL; ++i) *reinterpret_cast<uint4*>(st + BM * 128 + i * R::RB) = make_uint4(0, 0, 0, 0);
  };
  // Fragments of one 32-wide k-step (ks) of a stage, read from LDS into registers.
  auto read_frags = [&](const char* st, int ks, Frag<bf16_t> (&fa)[R::FM], Frag<bf16_t> (&fb)[R::FN]) {
    const int kc = ks * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < R::FM; ++i) {
      const int row = wm * R::WM + i * 16 + (lane & 15);
      fa[i].v[0] = *reinterpret_cast<const uint4*>(st + row * 128 + ((kc ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < R::FN; ++j) {
      const int row = wn * (BN / 2) + j * 16 + (lane & 15);
      fb[j].v[0] = *reinterpret_cast<const uint4*>(st + BM * 128 + row * 128 + ((kc ^ ((row >> 1) & 7)) << 4));
    }
  };
  auto mfmas = [&](const Frag<bf16_t> (&fa)[R::FM], const Frag<bf16_t> (&fb)[R::FN]) {
#pragma unroll
    for (int i = 0; i < R::FM; ++i)
#pragma unroll
      for (int j = 0; j < R::FN; ++j) mma(acc[i][j], fa[i], fb[j]);
  };
  // The same MFMAs with the LPS load instructions of stage `kt` spread between
  // them: a wave issuing its loads back to back stalls on the CU's shared load
  // path, while between MFMAs the issue hides under MFMA execution.
  constexpr int NM = R::FM * R::FN;
  constexpr int EVERY = NM / R::LPS > 0 ? NM / R::LPS : 1;
  auto mfmas_issue = [&](const Frag<bf16_t> (&fa)[R::FM], const Frag<bf16_t> (&fb)[R::FN], bool do_issue, int kt,
                         char* buf) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      mma(acc[m / R::FN][m % R::FN], fa[m / R::FN], fb[m % R::FN]);
      if (do_issue && (m + 1) % EVERY == 0 && (m + 1) / EVERY <= R::LPS) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(kt, buf, (m + 1) / EVERY - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_issue)
#pragma unroll
      for (int idx = NM / EVERY; idx < R::LPS; ++idx) issue_one(kt, buf, idx);
  };
  // Stage kt's data is in LDS for every wave, and every wave has finished
  // reading the buffer that the next issue refills. A plain barrier:
  // __syncthreads() would also wait for the loads in flight for later stages.
  auto stage_ready = [&](int kt, char* buf) {
    wait_vmcnt(min(NS - 2, nk - 1 - kt) * R::LPS);  // this wave's loads of stage kt landed
    zero_tail(kt, buf);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // Software pipeline: the barrier of stage kt+1 sits between the two k-steps
  // of stage kt, so the first fragments of stage kt+1 stream out of LDS while
  // the second k-step of stage kt runs on the MFMA units.
  Frag<bf16_t> fa0[R::FM], fb0[R::FN], fa1[R::FM], fb1[R::FN];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, L[s]);
  stage_ready(0, L[0]);
  if (NS - 1 < nk) issue(NS - 1, L[NS - 1]);
  read_frags(L[0], 0, fa0, fb0);
  for (int kt0 = 0; kt0 < nk; kt0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kt = kt0 + s;
      if (kt >= nk) break;
      read_frags(L[s], 1, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      bool refill = false;
      if (kt + 1 < nk) {
        stage_ready(kt + 1, L[(s + 1) % NS]);
        refill = kt + NS < nk;  // stage kt+NS goes into the buffer stage kt just left
        read_frags(L[(s + 1) % NS], 0, fa0, fb0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas_issue(fa1, fb1, refill, kt + NS, L[s]);
    }
  }
  __syncthreads();
}

// Writes the accumulators of rows [c*CR, c*CR+CR) into the fp32 LDS tile.
template <typename T, int BM, int BN, int NW = 4, typename S = GemmShape<T, BM, BN, NW>>
__device__ __forceinline__ void acc_to_lds(const f32x4 (&acc)[S::FM][S::FN], float* Cs, int c) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    const int r0 = wm * S::WM + i * 16;  // first row of this fragment
    if (r0 / S::CR != c) continue;
    const int rb = r0 - c * S::CR;
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(rb + (lane >> 4) * 4 + r) * S::EPI_LD + wn * S::WN + j * 16 + (lane & 15)] = acc[i][j][r];
  }
}


// ---------------------------------------------------------------------------
// bf16 256x256 tiles on eight waves in two groups of four ("ping-pong").
//
// The k loop walks 64-wide blocks of the A and B rows (128 bytes per row, in
// the row layout, chunk swizzle and per-wave load slots of LdsRing<256, 256,
// 2, 8>, held in the five-slot ring below). Group g (waves 4g..4g+3, one on
// each SIMD) owns tile rows 128g..128g+127; its wave q
// owns columns 64q..64q+63, a 128x64 wave tile of 8x4 16x16 fragments. Each
// block is used in two 32-wide half-steps. In every half-step a group first
// reads that half-step's fragments from LDS into registers (memory phase) and
// then runs its 32 MFMAs from registers only (compute phase). The two groups
// are one phase apart, so on each SIMD one wave issues MFMAs while the other
// waits on LDS, and a workgroup barrier separates the phases.
//
// Why this shape: a CU pulls global->LDS data at a fixed rate of cache-line
// requests (about 0.44 lines per clock), so the bytes per MFMA of the tile set
// the ceiling. A 256x256 tile needs 64 KB per 64-k block for 8.4 MFLOP, against
// 40 KB for 3.1 MFLOP with a 192x128 tile. 128-byte row segments keep each
// request a whole line (64-byte segments halve the rate).
//
// Every wave waits for its own loads of block j+1 and zeroes its chunks past K
// before the barrier that opens block j+1's first memory phase.
// ---------------------------------------------------------------------------
using PPRing = LdsRing<256, 256, 2, 8>;

// 32 KB slots of the ping-pong ring: five of them (all 160 KB of a CU's LDS).
// Part p of the k loop (p = 2j: the 256 A rows of 64-k block j, p = 2j + 1:
// its 256 B rows; 128 bytes per row) lives in slot p % 5. A slot is refilled
// once both groups have read the part five before it. Every wave issues B of
// block j + 1 at the first half-step of block j and A of block j + 2 at the
// second, so up to 96 KB are in flight while block j is multiplied.
constexpr int PP_SLOT = 256 * 128;

template <bool HALF>
__device__ __forceinline__ void gemm_mainloop_pp(f32x4 (&acc)[8][4], char* ring,
                                                 const bf16_t* (&ap)[PPRing::AL], const bf16_t* (&bp)[PPRing::BL],
                                                 int K, const bf16_t* adummy, const bf16_t* bdummy) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, q = wave & 3;
  const int kchunk = ((tid & 7) ^ ((tid >> 4) & 7)) * 8;  // logical k offset this lane loads
  const int nkb = (K + 63) >> 6;
  const int nh = 2 * nkb;
  const uint32_t rbase = (uint32_t)(uintptr_t)(lds_char*)ring + wave * 1024;

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto slot = [](int p) { return p % 5; };
  auto issue_a = [&](int kb) {
    const int k = kb * 64 + kchunk;
    const uint32_t st = rbase + slot(2 * kb) * PP_SLOT;
#pragma unroll
    for (int i = 0; i < PPRing::AL; ++i)
      dma16((ap[i] != nullptr && k < K) ? ap[i] + k : adummy, st + i * PPRing::RB);
  };
  auto issue_b = [&](int kb) {
    const int k = kb * 64 + kchunk;
    const uint32_t st = rbase + slot(2 * kb + 1) * PP_SLOT;
#pragma unroll
    for (int i = 0; i < PPRing::BL; ++i)
      dma16((bp[i] != nullptr && k < K) ? bp[i] + k : bdummy, st + i * PPRing::RB);
  };
  // This wave's loads of block kb are in LDS: the only loads issued after its
  // B rows are the A rows of block kb + 1 (vector-memory loads of a wave
  // complete in order). Chunks past K are then zeroed.
  auto land = [&](int kb) {
    if (kb + 1 < nkb) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kb * 64 + kchunk < K) return;
    char* sa = ring + slot(2 * kb) * PP_SLOT + tid * 16;
    char* sb = ring + slot(2 * kb + 1) * PP_SLOT + tid * 16;
#pragma unroll
    for (int i = 0; i < PPRing::AL; ++i) *reinterpret_cast<uint4*>(sa + i * PPRing::RB) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PPRing::BL; ++i) *reinterpret_cast<uint4*>(sb + i * PPRing::RB) = make_uint4(0, 0, 0, 0);
  };
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const int lrow = lane & 15, sw = (lrow >> 1) & 7;
  Frag<bf16_t> fa[8], fb[4];

  issue_a(0);
  issue_b(0);
  if (1 < nkb) issue_a(1);
  land(0);
  bar();
  if (g == 1) bar();
  for (int h = 0; h < nh; ++h) {
    const int kb = h >> 1;
    // memory phase: this half-step's fragment reads, then (after them, so
    // the reads start first) B of block kb + 1 at the first half-step and A
    // of block kb + 2 at the second
    {
      const char* sa = ring + slot(2 * kb) * PP_SLOT;
      const char* sb = ring + slot(2 * kb + 1) * PP_SLOT;
      const int off = lrow * 128 + ((((h & 1) * 4 + (lane >> 4)) ^ sw) << 4);
      // B first: the first MFMAs need only the B fragments and one A fragment
      if (!HALF || g == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j].v[0] = *reinterpret_cast<const uint4*>(sb + (64 * q + 16 * j) * 128 + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[i].v[0] = *reinterpret_cast<const uint4*>(sa + (128 * g + 16 * i) * 128 + off);
      }
    }
    if (!(h & 1)) {
      if (kb + 1 < nkb) issue_b(kb + 1);
    } else {
      if (kb + 2 < nkb) issue_a(kb + 2);
    }
    // Group 1's reads of a block's second half are the block's last: they
    // must land before the barrier after which its slots are refilled. Other
    // reads may still be in flight (each MFMA waits for its own fragments).
    if (g == 1 && (h & 1)) {
      if (kb + 1 < nkb) land(kb + 1);
      bar();
    } else {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    // compute phase
    __builtin_amdgcn_s_setprio(1);
    if (!HALF || g == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (g == 0 && (h & 1) && kb + 1 < nkb) land(kb + 1);
    bar();
  }
  if (g == 0) bar();
}

// ============================================================== dense GEMM
template <typename T, int BM, int BN, bool TWO, int NS, int NW>
__global__ __launch_bounds__(NW * 64, (NW == 8 && BM * BN <= 16384) ? 4 : 1) void k_dense_gemm(DenseGemm g) {
  static_assert(sizeof(T) == 2 || NW == 4, "the fp32 path runs four waves");
  using S = GemmShape<T, BM, BN, NW>;
  static_assert(BM != 256 || (sizeof(T) == 2 && BN == 256 && NW == 8 && !TWO), "256x256 tiles: bf16, one K phase");
  const int Mact = g.Mdev ? *g.Mdev : g.M;
  int ntot = 0;
  for (int s = 0; s < g.nseg; ++s) ntot += g.seg[s].ncols;
  const int ntn = (ntot + BN - 1) / BN;
  // Tiles of the active rows only (the grid covers M; compacted rows may be
  // fewer), spread over the XCDs by dispatch order. Each XCD's share is walked
  // in groups of GM row tiles, column block by column block, so the tiles an
  // XCD runs together share both A rows and B columns in its L2 (measured in
  // place against walking whole columns: -1.6 to -2.6 % on the large forwards).
  constexpr int GM = 4;
  const int ntm = ((Mact < g.M ? Mact : g.M) + BM - 1) / BM;
  const int nb = ntm * ntn;
  if ((int)blockIdx.x >= nb) return;
  const int L = xcd_remap(blockIdx.x, nb);
  const int gfirst = (L / (GM * ntn)) * GM, gr = L % (GM * ntn);
  const int gsz = ntm - gfirst < GM ? ntm - gfirst : GM;
  const int mt = gfirst + gr % gsz, nt = gr / gsz;
  const int m0 = mt * BM, n0 = nt * BN;
  const int z = blockIdx.z;
  const int tid = threadIdx.x;

  const T* ap[S::A_LD];
  const T* bp[S::B_LD];
  const T* ap2[S::A_LD];
  const T* bp2[S::B_LD];
  const T* A = reinterpret_cast<const T*>(g.A) + (long long)z * g.a_bstride;
#pragma unroll
  for (int i = 0; i < S::A_LD; ++i) {
    const int r = (tid + i * S::NT) / S::VPR;
    const int row = m0 + r;
    ap[i] = nullptr;
    ap2[i] = nullptr;
    if (row < Mact) {
      const int src = (g.gather && g.rows) ? g.rows[row] : row;
      ap[i] = A + (long long)src * g.lda;
      if (TWO) ap2[i] = reinterpret_cast<const T*>(g.A2) + (long long)row * g.lda2;
    }
  }
  // 256x256 tiles with RoPE over 128-wide heads: wave q's 64 columns are dims
  // 32(q & 1) .. +31 of head q >> 1 and then their partners 64 dims on, so a
  // lane holds both members of its rotation pairs (64-wide heads already lie
  // that way: one head per wave, partners 32 columns apart)
  const bool perm128 = BM == 256 && g.seg[0].rope && g.rope_dim == 128;
#pragma unroll
  for (int i = 0; i < S::B_LD; ++i) {
    int r = (tid + i * S::NT) / S::VPR;
    if (perm128) r = 128 * (r >> 7) + 32 * ((r >> 6) & 1) + (r & 31) + ((r & 32) ? 64 : 0);
    const int c = n0 + r;
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

  if constexpr (BM == 256) {
    // 256x256 ping-pong tiles (the expert GEMMs' main loop) for one B segment
    // whose rows are stored in place or scattered to their token, with or
    // without RoPE over 64- or 128-wide heads (no depth RoPE, no cache rows:
    // the host's rule). Each wave writes its 128 x 64 outputs through its own
    // LDS slice (fp32, 64 rows per pass), no workgroup barrier.
    __shared__ __align__(16) char ring[5 * PP_SLOT];
    const T* bd = reinterpret_cast<const T*>(g.seg[0].B) + (long long)z * g.b_bstride;
    f32x4 acc[8][4];
    gemm_mainloop_pp<false>(acc, ring, ap, bp, g.K, A, bd);
    constexpr int P = 68;
    static_assert(64 * P * 4 <= 5 * PP_SLOT / 8, "staging exceeds the wave's slice");
    const int lane = tid & 63, wave = tid >> 6, wg = wave >> 2, wq = wave & 3;
    float* sf = reinterpret_cast<float*>(ring + wave * (5 * PP_SLOT / 8));
    const GemmSeg& sg = g.seg[0];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sf[(16 * i + 4 * (lane >> 4) + r) * P + 16 * j + (lane & 15)] = acc[4 * half + i][j][r];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (!sg.rope) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int v = lane + 64 * it, row = v >> 3, c8 = v & 7;
          const int m = m0 + 128 * wg + 64 * half + row, col = n0 + 64 * wq + 8 * c8;
          const float4 x0 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c8);
          const float4 x1 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c8 + 4);
          const float vv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          if (m < Mact && col < ntot) {
            const long long orow = sg.scatter && g.rows ? g.rows[m] : m;
            const long long off = (long long)z * g.c_bstride + orow * sg.ldc + col;
            if (sg.out_f32) store8<float>(reinterpret_cast<float*>(sg.C) + off, vv);
            else store8<T>(reinterpret_cast<T*>(sg.C) + off, vv);
          }
        }
      } else {
        // RoPE: lane item (row, c4) takes 8 dims j .. j+7 of the first half of
        // a head (staged columns 8c4 ..) and their partners j + rh .. (staged
        // 32 columns on); same arithmetic as the smaller tiles' epilogue
        const int rh = g.rope_dim >> 1;  // 32 or 64
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int v = lane + 64 * it, row = v >> 2, c4 = v & 3;
          const int m = m0 + 128 * wg + 64 * half + row;
          const int jj = (rh == 64 ? 32 * (wq & 1) : 0) + 8 * c4;  // dim inside the half
          const int colA = n0 + (rh == 64 ? 128 * (wq >> 1) : 64 * wq) + jj, colB = colA + rh;
          const float* xa = sf + row * P + 8 * c4;
          const float* xb = xa + 32;
          if (m < Mact && colB < ntot) {
            const int tok = g.rows ? g.rows[m] : m;
            const long long orow = sg.scatter ? tok : m;
            const int pp = g.pos_dev ? *g.pos_dev : tok % g.seq;
            const float4 c0 = *reinterpret_cast<const float4*>(g.cosb + pp * rh + jj);
            const float4 c1 = *reinterpret_cast<const float4*>(g.cosb + pp * rh + jj + 4);
            const float4 s0 = *reinterpret_cast<const float4*>(g.sinb + pp * rh + jj);
            const float4 s1 = *reinterpret_cast<const float4*>(g.sinb + pp * rh + jj + 4);
            const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            float va[8], vb[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              va[x] = xa[x] * cs[x] - xb[x] * sn[x];
              vb[x] = xa[x] * sn[x] + xb[x] * cs[x];
            }
            const long long off = (long long)z * g.c_bstride + orow * sg.ldc;
            if (sg.out_f32) {
              store8<float>(reinterpret_cast<float*>(sg.C) + off + colA, va);
              store8<float>(reinterpret_cast<float*>(sg.C) + off + colB, vb);
            } else {
              store8<T>(reinterpret_cast<T*>(sg.C) + off + colA, va);
              store8<T>(reinterpret_cast<T*>(sg.C) + off + colB, vb);
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    return;
  } else {
  constexpr int ST = sizeof(T) == 2 ? LdsRing<BM, BN, NS, NW>::STAGE : S::SMEM;
  __shared__ __align__(16) char L0[ST];
  __shared__ __align__(16) char L1[sizeof(T) == 2 ? ST : 16];
  __shared__ __align__(16) char L2[sizeof(T) == 2 && NS > 2 ? ST : 16];
  __shared__ __align__(16) char L3[sizeof(T) == 2 && NS > 3 ? ST : 16];
  char* smem = L0;
  f32x4 acc[S::FM][S::FN];
  if constexpr (sizeof(T) == 2) {
    const T* bd = reinterpret_cast<const T*>(g.seg[0].B) + (long long)z * g.b_bstride;
    char* const Ls[4] = {L0, L1, L2, L3};
    char* const (&Lr)[NS] = *reinterpret_cast<char* const(*)[NS]>(Ls);
    gemm_mainloop_ring<BM, BN, NS, TWO, NW>(acc, Lr, ap, bp, g.K, ap2, bp2, g.K2, A, bd,
                                        reinterpret_cast<const T*>(g.A2), reinterpret_cast<const T*>(g.B2));
  } else {
    gemm_mainloop<T, BM, BN, TWO>(acc, smem, ap, bp, g.K, ap2, bp2, g.K2);
  }

  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int c = 0; c < BM / S::CR; ++c) {
    acc_to_lds<T, BM, BN, NW>(acc, Cs, c);
    lds_barrier();
    const int rbase = m0 + c * S::CR;
    const int nrows = S::CR;
    if (g.epi == EPI_STORE) {
      for (int idx = tid; idx < nrows * (BN / 8); idx += S::NT) {
        const int r = idx / (BN / 8), c8 = (idx % (BN / 8)) * 8;
        const int row = rbase + r, gc = n0 + c8;
        if (row >= Mact || gc >= ntot) continue;
        int s = 0, base = 0;
        while (s + 1 < g.nseg && gc >= base + g.seg[s].ncols) { base += g.seg[s].ncols; ++s; }
        const GemmSeg& sg = g.seg[s];
        const int lc = gc - base;
        const int tok = g.rows ? g.rows[row] : row;
        const long long orow = sg.row_mul ? (long long)tok * sg.row_mul + *g.pos_dev : (sg.scatter ? tok : row);
        const float* crow = Cs + r * S::EPI_LD;
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x];
        const int rhalf = g.rope_dim >> 1;
        // whole-vector RoPE: the 8 columns lie in one half of one head and
        // share one rotation position, so their angle entries are 8
        // consecutive table floats (same arithmetic as the per-element form)
        const bool rope_vec = sg.rope && (rhalf & 7) == 0 && (!g.drope || ((rhalf >> 1) & 7) == 0);
        if (rope_vec) {
          const int hd0 = lc % g.rope_dim, jj0 = hd0 % rhalf;
          const int pp = g.drope ? (jj0 < (rhalf >> 1) ? g.dpos0 : g.dpos1) : (g.pos_dev ? *g.pos_dev : tok % g.seq);
          const float4 c0 = *reinterpret_cast<const float4*>(g.cosb + pp * rhalf + jj0);
          const float4 c1 = *reinterpret_cast<const float4*>(g.cosb + pp * rhalf + jj0 + 4);
          const float4 s0 = *reinterpret_cast<const float4*>(g.sinb + pp * rhalf + jj0);
          const float4 s1 = *reinterpret_cast<const float4*>(g.sinb + pp * rhalf + jj0 + 4);
          const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          if (hd0 < rhalf) {
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x] * cs[x] - crow[c8 + x + rhalf] * sn[x];
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x - rhalf] * sn[x] + crow[c8 + x] * cs[x];
          }
        } else if (sg.rope) {
          const int rd = g.rope_dim, half = rd >> 1;
          const int pos = g.pos_dev ? *g.pos_dev : tok % g.seq;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int hd = (lc + x) % rd;
            const int jj = hd % half;
            const int pp = g.drope ? (jj < (half >> 1) ? g.dpos0 : g.dpos1) : pos;
            const float cs = g.cosb[pp * half + jj], sn = g.sinb[pp * half + jj];
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
    lds_barrier();
  }
  }
}

template <typename T, int BM, int BN, int NS, int NW = 4>
static hipError_t dense_launch(const DenseGemm& g, hipStream_t s) {
  int ntot = 0;
  for (int i = 0; i < g.nseg; ++i) ntot += g.seg[i].ncols;
  const int ntn = (ntot + BN - 1) / BN, ntm = (g.M + BM - 1) / BM;
  dim3 grid(ntn * ntm, 1, g.batch > 0 ? g.batch : 1);
  if (g.A2) {
    if constexpr (BM == 256) return hipErrorInvalidValue;  // one K phase only
    else hipLaunchKernelGGL((k_dense_gemm<T, BM, BN, true, NS, NW>), grid, dim3(NW * 64), 0, s, g);
  } else {
    hipLaunchKernelGGL((k_dense_gemm<T, BM, BN, false, NS, NW>), grid, dim3(NW * 64), 0, s, g);
  }
  return hipGetLastError();
}

template <typename T, int BM, int BN>
static hipError_t dense_ns(const DenseGemm& g, hipStream_t s) {
  if (sizeof(T) == 4) return dense_launch<T, BM, BN, 2>(g, s);  // fp32 ignores the stage count
  switch (g.ns) {
    case 3: return dense_launch<T, BM, BN, 3>(g, s);
    case 4: return dense_launch<T, BM, BN, 4>(g, s);
    // a few rows (one-token decode): a four-stage ring, the grid is small;
    // 64x64 tiles: three stages (measured in place on the gqa forward)
    default:
      if (g.M <= 64) return dense_launch<T, BM, BN, 4>(g, s);
      if (BM == 64 && BN == 64) return dense_launch<T, BM, BN, 3>(g, s);
      return dense_launch<T, BM, BN, 2>(g, s);
  }
}

template <typename T>
static hipError_t dense_dispatch(const DenseGemm& g, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (g.nw == 8) {  // eight waves: 64x64 tiles with three stages, 128x128 with two, 256x256 ping-pong
      if (g.bm == 256 && g.bn == 256) {
        const GemmSeg& sg = g.seg[0];
        if (g.A2 || g.nseg != 1 || g.epi != EPI_STORE || sg.row_mul) return hipErrorInvalidValue;
        if (sg.rope && (g.drope || (g.rope_dim != 64 && g.rope_dim != 128) || sg.ncols % g.rope_dim ||
                        !g.cosb || !g.sinb || (!g.pos_dev && g.seq <= 0)))
          return hipErrorInvalidValue;
        return dense_launch<T, 256, 256, 2, 8>(g, s);
      }
      if (g.bm == 64 && g.bn == 64) return dense_launch<T, 64, 64, 3, 8>(g, s);
      if (g.bm == 128 && g.bn == 128) return dense_launch<T, 128, 128, 2, 8>(g, s);
      return hipErrorInvalidValue;
    }
  }
  if (g.bm == 64 && g.bn == 64) return dense_ns<T, 64, 64>(g, s);
  if (g.bm == 64 && g.bn == 128) return dense_ns<T, 64, 128>(g, s);
  if (g.bm == 128 && g.bn == 64) return dense_ns<T, 128, 64>(g, s);
  return dense_ns<T, 128, 128>(g, s);
}

hipError_t launch_dense_gemm(const DenseGemm& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  return g.dtype == DT_F32 ? dense_dispatch<float>(g, s) : dense_dispatch<bf16_t>(g, s);
}

// ============================================================ grouped GEMM
template <typename T, int BM, int BN, int KIND, int NS, int NW>
__global__ __launch_bounds__(NW * 64, (NW == 8 && BM * BN <= 16384) ? 4 : 1) void k_grouped_gemm(GroupedGemm g) {
  static_assert(sizeof(T) == 2 || NW == 4, "the fp32 path runs four waves");
  using S = GemmShape<T, BM, BN, NW>;
  const int G = g.E + g.Se;
  const int n = g.ndev ? *g.ndev : g.n_static;
  // KIND 0 produces BN/2 SwiGLU outputs per tile from BN/2 gate + BN/2 up rows
  const int OUTW = KIND == 0 ? BN / 2 : BN;
  const int ntn = (g.N + OUTW - 1) / OUTW;
  // Tile schedule from the per-expert counts: expert g (routed: cnt[g] rows;
  // shared: n rows) owns ceil(rows / BM) consecutive m-tiles. The grid is
  // sized for the worst case; only the first total_mt * ntn blocks have a
  // tile. Those are spread over the XCDs by dispatch order, and each XCD's
  // share is remapped to consecutive tiles (an order chosen below).
  const int lane = threadIdx.x & 63;
  auto rows_of = [&](int gg) { return gg < G ? (gg < g.E ? g.cnt[gg] : n) : 0; };
  auto scan = [&](int v) {  // inclusive prefix sum over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(v, o, 64);
      if (lane >= o) v += y;
    }
    return v;
  };
  int total_mt = 0;
  for (int b0 = 0; b0 < G; b0 += 64) total_mt += __shfl(scan((rows_of(b0 + lane) + BM - 1) / BM), 63, 64);
  const int nb = total_mt * ntn;
  if ((int)blockIdx.x >= nb) return;
  const int L = xcd_remap(blockIdx.x, nb);
  const int q = L / ntn;  // expert of tile L: the one whose m-tiles hold q
  // this tile's expert, its first tile and the first output row of its rows
  int grp = -1, tstart = 0, rbase = 0, tlg = 1;
  for (int b0 = 0, ct = 0, cr = 0; b0 < G && grp < 0; b0 += 64) {
    const int gg = b0 + lane, rows = rows_of(gg), tl = (rows + BM - 1) / BM;
    const int it = scan(tl), ir = scan(gg < g.E ? rows : 0);
    const int end = ct + it;
    const unsigned long long hit = __ballot(gg < G && q >= end - tl && q < end);
    if (hit) {
      const int w = __ffsll((long long)hit) - 1;
      grp = b0 + w;
      tstart = __shfl(end - tl, w, 64);
      tlg = __shfl(tl, w, 64);
      rbase = cr + __shfl(ir - (gg < g.E ? rows : 0), w, 64);
    }
    ct += __shfl(it, 63, 64);
    cr += __shfl(ir, 63, 64);
  }
  grp = __builtin_amdgcn_readfirstlane(grp);
  // Order of an expert's tiles [tstart * ntn, (tstart + tlg) * ntn) in L.
  // 64-row down tiles (an expert has few rows, hence few m-tiles): m-tiles
  // innermost, so the m-tiles that stream one weight slab run side by side on
  // one XCD and share it in L2. Gate/up: the n-tiles in bands of GUB, each
  // band walked m-tile by m-tile with its n-tiles innermost. Tiles that share
  // A rows start together, and so do (GUB tiles apart) tiles that share weight
  // rows; L2 keeps data only for a few of the 32 k-stages of a tile, so tiles
  // that start far apart fetch shared operands again (wide MoE shape, 256x256
  // tiles: 2.7 GB fetched per launch with n-tiles innermost, 1.64 GB with
  // bands of 2, 1.46 GB with bands of 4, 1.61 GB with bands of 8, the last
  // three equally fast). Otherwise n-tiles innermost.
  int mt, nt;
  if constexpr (KIND == 1 && BM == 64) {
    const int r = L - tstart * ntn;
    nt = r / tlg;
    mt = tstart + r % tlg;
  } else if constexpr (KIND == 0) {
    constexpr int GUB = 4;
    const int r = L - tstart * ntn;
    const int band = r / (tlg * GUB), rem = r % (tlg * GUB);
    const int bsz = ntn - band * GUB < GUB ? ntn - band * GUB : GUB;
    mt = tstart + rem / bsz;
    nt = band * GUB + rem % bsz;
  } else {
    mt = q;
    nt = L % ntn;
  }
  const bool routed = grp < g.E;
  const int rows_g = routed ? g.cnt[grp] : n;
  const int pbase = routed ? rbase : n * g.k + (grp - g.E) * n;
  const int ml0 = (mt - tstart) * BM;
  const int n0 = nt * OUTW;
  const int tid = threadIdx.x;
  const T* A = reinterpret_cast<const T*>(g.A);

  const T* ap[S::A_LD];
  const T* bp[S::B_LD];
#pragma unroll
  for (int i = 0; i < S::A_LD; ++i) {
    const int m = ml0 + (tid + i * S::NT) / S::VPR;
    ap[i] = nullptr;
    if (m < rows_g) {
      int src;
      if (KIND == 0) src = routed ? g.pcap[(long long)grp * g.cap + m] : m;
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
      const int c = (tid + i * S::NT) / S::VPR;
      // 256x256 tiles: wave q's 64 columns are the gate then the up rows of
      // features n0 + 32q .. +31, so one lane holds both halves of an output;
      // other tiles: the gate rows of the BN/2 features, then their up rows
      const bool up = BM == 256 ? ((c & 63) >= 32) : (c >= BN / 2);
      const int f = n0 + (BM == 256 ? 32 * (c >> 6) + (c & 31) : c % (BN / 2));
      bp[i] = f < g.N ? ((up ? wu : wg) + (long long)f * g.K) : nullptr;
    }
  } else {
    const T* wd = reinterpret_cast<const T*>(routed ? g.W1 : g.S1) + (routed ? grp : grp - g.E) * wsz;
#pragma unroll
    for (int i = 0; i < S::B_LD; ++i) {
      const int c = n0 + (tid + i * S::NT) / S::VPR;
      bp[i] = c < g.N ? wd + (long long)c * g.K : nullptr;
    }
  }

  if constexpr (BM == 256) {  // 256x256 ping-pong tiles (bf16, eight waves, no K slices)
    const T* bd = bp[0] ? bp[0] : reinterpret_cast<const T*>(routed ? g.W1 : g.S1);
    const int Kl = g.K;
    __shared__ __align__(16) char ring[5 * PP_SLOT];
    f32x4 acc[8][4];
    // an expert's last tile with at most 128 rows of data: group 1's half of
    // the tile holds none, so it skips its fragment reads and MFMAs (a
    // separate instantiation keeps both loops free of branches)
    if (rows_g - ml0 <= 128) gemm_mainloop_pp<true>(acc, ring, ap, bp, Kl, A, bd);
    else gemm_mainloop_pp<false>(acc, ring, ap, bp, Kl, A, bd);
    // Epilogue, wave by wave (no workgroup barrier): the wave's outputs go
    // through its own 20 KB slice of the ring (free once every wave has passed
    // the loop's last barrier) as fp32 (whole-dword LDS writes; single bf16
    // writes measured 2.5 % slower on the down projection) and leave as
    // 16-byte bf16 row vectors. Rows of the wave: tile rows 128g .. 128g + 127.
    constexpr int WSLICE = 5 * PP_SLOT / 8;
    const int lane = tid & 63, wave = tid >> 6, wg = wave >> 2, wq = wave & 3;
    char* wbuf = ring + wave * WSLICE;
    auto wave_lds_sync = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
    if constexpr (KIND == 0) {
      // SwiGLU of features n0 + 32wq .. +31: fragments 0, 1 hold the gate and
      // 2, 3 the up projections of the same 16-feature columns
      constexpr int P = 36;  // fp32 staging row pitch (full-dword LDS writes)
      static_assert(128 * P * 4 <= WSLICE, "SwiGLU staging exceeds the wave's slice");
      float* sf = reinterpret_cast<float*>(wbuf);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[i][jj][r], up = acc[i][jj + 2][r];
            sf[(16 * i + 4 * (lane >> 4) + r) * P + 16 * jj + (lane & 15)] = silu_mul(gt, up);
          }
      wave_lds_sync();
      T* C = reinterpret_cast<T*>(g.C);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int v = lane + 64 * it, row = v >> 2, c4 = v & 3;
        const int m = ml0 + 128 * wg + row, f = n0 + 32 * wq + 8 * c4;
        const float4 x0 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c4);
        const float4 x1 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c4 + 4);
        const float vv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        if (m < rows_g && f < g.N) store8<T>(C + (long long)(pbase + m) * g.ldc + f, vv);
      }
    } else {
      // fp32 staging (full-dword LDS writes), 64 rows per pass
      constexpr int P = 68;
      static_assert(64 * P * 4 <= WSLICE, "output staging exceeds the wave's slice");
      float* sf = reinterpret_cast<float*>(wbuf);
      T* C = reinterpret_cast<T*>(g.C);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              sf[(16 * i + 4 * (lane >> 4) + r) * P + 16 * j + (lane & 15)] = acc[4 * half + i][j][r];
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int v = lane + 64 * it, row = v >> 3, c8 = v & 7;
          const int m = ml0 + 128 * wg + 64 * half + row, col = n0 + 64 * wq + 8 * c8;
          const float4 x0 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c8);
          const float4 x1 = *reinterpret_cast<const float4*>(sf + row * P + 8 * c8 + 4);
          const float vv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          if (m < rows_g && col < g.N) store8<T>(C + (long long)(pbase + m) * g.ldc + col, vv);
        }
        wave_lds_sync();
      }
    }
    return;
  } else {
  constexpr int ST = sizeof(T) == 2 ? LdsRing<BM, BN, NS, NW>::STAGE : S::SMEM;
  __shared__ __align__(16) char L0[ST];
  __shared__ __align__(16) char L1[sizeof(T) == 2 ? ST : 16];
  __shared__ __align__(16) char L2[sizeof(T) == 2 && NS > 2 ? ST : 16];
  __shared__ __align__(16) char L3[sizeof(T) == 2 && NS > 3 ? ST : 16];
  char* smem = L0;
  f32x4 acc[S::FM][S::FN];
  if constexpr (sizeof(T) == 2) {
    const T* bd = bp[0] ? bp[0] : reinterpret_cast<const T*>(routed ? g.W1 : g.S1);
    char* const Ls[4] = {L0, L1, L2, L3};
    char* const (&Lr)[NS] = *reinterpret_cast<char* const(*)[NS]>(Ls);
    int Kl = g.K;
    if (KIND == 1 && gridDim.y > 1) {   // K slice blockIdx.y of gridDim.y (whole 64-wide stages)
      const int Ks = (((g.K + 63) / 64 + (int)gridDim.y - 1) / (int)gridDim.y) * 64;
      const int k0 = (int)blockIdx.y * Ks;
      Kl = g.K - k0 < Ks ? g.K - k0 : Ks;
#pragma unroll
      for (int i = 0; i < S::A_LD; ++i)
        if (ap[i]) ap[i] += k0;
#pragma unroll
      for (int i = 0; i < S::B_LD; ++i)
        if (bp[i]) bp[i] += k0;
    }
    gemm_mainloop_ring<BM, BN, NS, false, NW>(acc, Lr, ap, bp, Kl, ap, bp, 0, A, bd, A, bd);
  } else {
    gemm_mainloop<T, BM, BN, false>(acc, smem, ap, bp, g.K, ap, bp, 0);
  }

  float* Cs = reinterpret_cast<float*>(smem);
  T* C = reinterpret_cast<T*>(g.C);
#pragma unroll 1
  for (int c = 0; c < BM / S::CR; ++c) {
    acc_to_lds<T, BM, BN, NW>(acc, Cs, c);
    lds_barrier();
    const int nrows = S::CR;
    for (int idx = tid; idx < nrows * (OUTW / 8); idx += S::NT) {
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
          v[x] = silu_mul(gt, up);
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = crow[c8 + x];
      }
      if (KIND == 1 && gridDim.y > 1)
        store8<float>(g.part + (long long)blockIdx.y * g.pstride + (long long)(pbase + m) * g.ldc + col, v);
      else
        store8<T>(C + (long long)(pbase + m) * g.ldc + col, v);
    }
    lds_barrier();
  }
  }
}

template <typename T, int BM, int BN, int KIND, int NS, int NW = 4>
static hipError_t grouped_launch(const GroupedGemm& g, hipStream_t s) {
  const int outw = KIND == 0 ? BN / 2 : BN;
  const int ntn = (g.N + outw - 1) / outw;
  dim3 grid(g.max_mtiles * ntn, KIND == 1 && sizeof(T) == 2 && g.ksplit > 1 ? g.ksplit : 1);
  hipLaunchKernelGGL((k_grouped_gemm<T, BM, BN, KIND, NS, NW>), grid, dim3(NW * 64), 0, s, g);
  return hipGetLastError();
}

template <typename T>
static hipError_t grouped_dispatch(const GroupedGemm& g, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    return g.kind == 0 ? grouped_launch<T, GU_BM, GU_BN, 0, 2>(g, s) : grouped_launch<T, DN_BM, DN_BN, 1, 2>(g, s);
  } else {
    // four waves: eight-wave expert tiles were slower in place (192x128 spills
    // at the register budget of two workgroups per CU; 128x128 needs more tiles)
#define RDT_G(K, BM, BN, NS) \
    if (g.kind == K && g.bm == BM && g.bn == BN && g.ns == NS) return grouped_launch<T, BM, BN, K, NS>(g, s);
    RDT_G(0, 64, 64, 3) RDT_G(0, 128, 128, 2) RDT_G(0, 160, 128, 2) RDT_G(0, 192, 128, 2)
    RDT_G(1, 64, 32, 3) RDT_G(1, 64, 64, 3) RDT_G(1, 64, 64, 4) RDT_G(1, 192, 128, 2)
#undef RDT_G
    // 256x256 ping-pong tiles: eight waves, one workgroup per CU, no K slices
    if (g.bm == 256 && g.bn == 256 && g.ns == 2) {
      if (g.ksplit > 1) return hipErrorInvalidValue;
      return g.kind == 0 ? grouped_launch<T, 256, 256, 0, 2, 8>(g, s) : grouped_launch<T, 256, 256, 1, 2, 8>(g, s);
    }
    return hipErrorInvalidValue;
  }
}

hipError_t launch_grouped_gemm(const GroupedGemm& g, hipStream_t s) {
  if (g.max_mtiles <= 0) return hipSuccess;
  if (g.ksplit > 1 && (g.kind != 1 || g.dtype != DT_BF16 || !g.part || g.ksplit > (g.K + 63) / 64))
    return hipErrorInvalidValue;
  return g.dtype == DT_F32 ? grouped_dispatch<float>(g, s) : grouped_dispatch<bf16_t>(g, s);
}

}  // namespace rdt
