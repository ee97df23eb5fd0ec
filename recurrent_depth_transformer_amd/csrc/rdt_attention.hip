// Causal flash attention for grouped-query and absorbed multi-latent attention.
//
// A workgroup of NW waves (4 or 8) owns one sequence b, NHB query heads that
// read the same kv head, and NW/NHB consecutive slices of QW query rows (rows
// of the compacted active list when ACT is on). Wave w handles head w % NHB
// and slice w / NHB. Key/value tiles of KT positions are shared by all waves:
// they are double-buffered in LDS, and the global loads of the next tile (of
// the next two, in two register sets, for 16-row slices) are in flight while
// the current tile is multiplied.
// Workgroups are numbered longest query tile first over the whole grid.
//
// The scores are formed transposed, S^T = K Q^T, so that a lane holds four
// consecutive keys of one query: that is exactly the k-slot layout the second
// MFMA needs for P, so O^T = V^T P^T is accumulated without moving P through
// LDS. In bf16, V stays row-major in LDS and the V^T fragments come from the
// LDS transpose read (ds_read_b64_tr_b16: within each 16-lane group, lane j
// receives element j & 3 of the 8-byte chunks addressed by lanes
// 4t + (j >> 2), t = 0..3). In fp32, V is written to LDS transposed.
//
// Multi-latent attention in absorbed form is the same computation with one kv
// head whose key is [c_kv | k_rope] and whose value is the c_kv prefix of the
// same row, shared by every query head; in bf16 (VK) the V^T fragments are
// then read from the K tile itself and no V tile is loaded. In that form the
// kernel also builds its queries (q_nope Wuk[h] on the MFMA, RoPE on q_pe) and
// applies the value up-projection Wuv[h] to its output rows, so neither the
// absorbed queries nor o_lat go through HBM.
#include "rdt_device.h"
#include "rdt_launch.h"

namespace rdt {


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Four 16-bit elements through the LDS transpose read (gfx950), as two dwords.
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

template <typename T, int DQK, int DV, int QW, int NHB, int KT, int NW, bool VK>
__global__ __launch_bounds__(NW * 64) void k_attention(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KB = KT / 16;  // 16-key blocks per tile
  constexpr int DQKP = (DQK + 31) / 32 * 32;
  constexpr int KS = DQKP / 32;
  constexpr int QS = QW / 16;
  constexpr int DS = DV / 16;
  constexpr int VEC = ST<T>::VEC;
  constexpr bool BF = sizeof(T) == 2;
  static_assert(!VK || (BF && DV <= DQK), "V from the K tile needs bf16 and DV <= DQK");
  constexpr int KLD = DQKP + VEC;
  // bf16: V row-major with rows padded by 16 (conflict-free transpose reads);
  // fp32: V transposed, rows of KT + 4 keys
  constexpr int VLD = BF ? DV + 16 : KT + 4;
  constexpr int VSZ = VK ? 8 : (BF ? KT * VLD : DV * VLD);
  constexpr int SLICES = NW / NHB;
  constexpr int BQ = QW * SLICES;  // query rows per workgroup (per head)
  // per-thread share of one K tile and one V tile (NT threads)
  constexpr int KV_VECS = KT * (DQKP / VEC);
  constexpr int KL = (KV_VECS + NT - 1) / NT;
  constexpr int VV = VK ? 0 : (BF ? KT * (DV / 8) : KT * (DV / 4));
  constexpr int VL = VV > 0 ? (VV + NT - 1) / NT : 1;
  __shared__ __align__(16) T Ks[2][KT * KLD];
  __shared__ __align__(16) T Vt[2][VSZ];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, lc = lane & 15;
  // linear workgroup id -> (query tile, sequence, head group), late query
  // tiles (the most keys) first
  const int nhg = a.H / NHB;
  const int bz = a.B * nhg;
  const int outer = (int)(blockIdx.x / bz);
  const bool split = a.dec && a.nsplit > 1;     // key range `outer` of a decode step
  const int qt = a.dec ? 0 : (int)(gridDim.x / bz) - 1 - outer;
  const int b = (blockIdx.x % bz) / nhg;
  const int h = (blockIdx.x % nhg) * NHB + (wave % NHB);
  const int slice = wave / NHB;
  const int kvh = (h * a.KV) / a.H;
  const int S = a.S;
  // token of query row x: its cache row in decode, else the token itself
  const int dpos = a.dec ? *a.dec_pos : 0;
  auto tok = [&](int x) { return a.dec ? (a.rows ? a.rows[x] : x) * S + dpos : (a.rows ? a.rows[x] : x); };
  const int seg0 = a.seg ? a.seg[b] : (a.dec ? b : b * S);
  const int seglen = a.seg ? a.seg[b + 1] - seg0 : (a.dec ? 1 : S);
  if (qt * BQ >= seglen) return;
  const int blk_first = seg0 + qt * BQ;
  const int blk_n = min(BQ, seglen - qt * BQ);
  const int last = blk_first + blk_n - 1;
  const int kmax = tok(last) - b * S + 1;  // keys 0..kmax-1
  const int qfirst = blk_first + slice * QW;
  const int nq = max(0, min(QW, blk_n - slice * QW));  // this wave's query rows

  const T* Q = reinterpret_cast<const T*>(a.q);
  const T* Kg = reinterpret_cast<const T*>(a.k);
  const T* Vg = reinterpret_cast<const T*>(a.v);
  const long long tokbase = (long long)b * S;

  int qpos[QS];
  Frag<T> qf[QS][KS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qq = qs * 16 + lc;
    const bool valid = qq < nq;
    const int i = qfirst + qq;
    qpos[qs] = valid ? tok(i) - b * S : -1;
    if constexpr (VK) continue;  // formed from q_nope and q_pe below
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 32 + lg * 8;
      if (valid && d0 < DQK)
        qf[qs][ks] = frag_lds<T>(Q + (long long)i * a.q_ld + (long long)h * a.q_hs + d0);
      else
        qf[qs][ks] = frag_zero<T>();
    }
  }

  f32x4 oacc[DS][QS];
  float mrow[QS], lrow[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    mrow[qs] = -INFINITY;
    lrow[qs] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) oacc[ds][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = a.scale * 1.4426950408889634f;  // exp2 domain
  // key tiles [kt_begin, nkt) of this workgroup
  int nkt = (kmax + KT - 1) / KT, kt_begin = 0;
  if (split) {
    const int per = (nkt + a.nsplit - 1) / a.nsplit;
    kt_begin = min(nkt, outer * per);
    nkt = min(nkt, kt_begin + per);
  }
  // first query position of this wave: tiles that end at or before it need
  // no causal mask
  int qlo = 0x7fffffff;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
    if (qpos[qs] >= 0) qlo = min(qlo, qpos[qs]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) qlo = min(qlo, __shfl_xor(qlo, o, 64));

  // ---- K/V tile: global -> registers -> LDS (fp32 V transposed); two
  // register sets so that two tiles can be in flight
  typedef uint4 RK[KL];
  typedef uint4 RV[VL];
  RK rk0, rk1;
  RV rv0, rv1;
  auto gload = [&](int k0, RK& rk, RV& rv) {
    if (k0 + KT <= kmax) {  // every key of the tile exists: loads without predicates
      const T* kb = Kg + (tokbase + k0) * a.k_ld + (long long)kvh * a.k_hs;
#pragma unroll
      for (int u = 0; u < KL; ++u) {
        const int v = tid + u * NT;
        const int kr = v / (DQKP / VEC), kc = (v % (DQKP / VEC)) * VEC;
        if ((KV_VECS % NT == 0 || v < KV_VECS) && (DQKP == DQK || kc < DQK))
          rk[u] = *reinterpret_cast<const uint4*>(kb + kr * a.k_ld + kc);
        else
          rk[u] = make_uint4(0, 0, 0, 0);
      }
      if constexpr (VK) return;
      const T* vb = Vg + (tokbase + k0) * a.v_ld + (long long)kvh * a.v_hs;
#pragma unroll
      for (int u = 0; u < VL; ++u) {
        const int v = tid + u * NT;
        const int kr = v / (DV / VEC), dc = (v % (DV / VEC)) * VEC;
        rv[u] = (VV % NT == 0 || v < VV) ? *reinterpret_cast<const uint4*>(vb + kr * a.v_ld + dc) : make_uint4(0, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KL; ++u) {
      const int v = tid + u * NT;
      const int kr = v / (DQKP / VEC), kc = (v % (DQKP / VEC)) * VEC;
      const int key = k0 + kr;
      rk[u] = (v < KV_VECS && key < kmax && kc < DQK)
                  ? *reinterpret_cast<const uint4*>(Kg + (tokbase + key) * a.k_ld + (long long)kvh * a.k_hs + kc)
                  : make_uint4(0, 0, 0, 0);
    }
    if constexpr (VK) return;
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int v = tid + u * NT;
      const int kr = v / (DV / VEC), dc = (v % (DV / VEC)) * VEC;
      const int key = k0 + kr;
      rv[u] = (v < VV && key < kmax)
                  ? *reinterpret_cast<const uint4*>(Vg + (tokbase + key) * a.v_ld + (long long)kvh * a.v_hs + dc)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf, const RK& rk, const RV& rv) {
#pragma unroll
    for (int u = 0; u < KL; ++u) {
      const int v = tid + u * NT;
      if (v < KV_VECS) {
        const int kr = v / (DQKP / VEC), kc = (v % (DQKP / VEC)) * VEC;
        *reinterpret_cast<uint4*>(&Ks[buf][kr * KLD + kc]) = rk[u];
      }
    }
    if constexpr (VK) return;
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int v = tid + u * NT;
      if (v >= VV) continue;
      if constexpr (BF) {
        const int kr = v / (DV / 8), dc = (v % (DV / 8)) * 8;
        *reinterpret_cast<uint4*>(&Vt[buf][kr * VLD + dc]) = rv[u];
      } else {
        const int kr = v / (DV / 4), dc = (v % (DV / 4)) * 4;
        const float* f = reinterpret_cast<const float*>(&rv[u]);
#pragma unroll
        for (int x = 0; x < 4; ++x) Vt[buf][(dc + x) * VLD + kr] = f[x];
      }
    }
  };

  auto tile = [&](int kt, int buf) {
    const int k0 = kt * KT;
    if (nq > 0) {
      const T* Kb = Ks[buf];
      const T* Vb = Vt[buf];
      // S^T[key][query] for 4 blocks of 16 keys
      f32x4 s[KB][QS];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[kb][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const Frag<T> kf = frag_lds<T>(Kb + (kb * 16 + lc) * KLD + ks * 32 + lg * 8);
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) mma(s[kb][qs], kf, qf[qs][ks]);
        }
      }
      // scale, causal mask (only on tiles that reach a query or the end of
      // the keys), online softmax (per query = per lane column)
      const bool masked = k0 + KT - 1 > qlo || k0 + KT > kmax;
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        float mx = -INFINITY;
        if (masked) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kp = k0 + kb * 16 + lg * 4 + r;
              float x = s[kb][qs][r];
              if (kp > qpos[qs] || kp >= kmax) x = -INFINITY;
              s[kb][qs][r] = x;
              mx = fmaxf(mx, x);
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qs][r]);
        }
        mx *= sc;  // scores stay raw; the scale (> 0) is applied inside the exponent
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // the reference max moves only when the tile's max exceeds it by more
        // than 8 (probabilities stay below 2^8); otherwise alpha is exactly 1
        const bool move = mx > mrow[qs] + 8.f;
        const float mnew = move ? mx : mrow[qs];
        const float base = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = move ? __builtin_amdgcn_exp2f(mrow[qs] - base) : 1.f;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qs][r], sc, -base));
            s[kb][qs][r] = p;
            rs += p;
          }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        lrow[qs] = lrow[qs] * alpha + rs;
        mrow[qs] = mnew;
        if (__ballot(move)) {  // some row's reference max moved
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) {
            oacc[ds][qs][0] *= alpha;
            oacc[ds][qs][1] *= alpha;
            oacc[ds][qs][2] *= alpha;
            oacc[ds][qs][3] *= alpha;
          }
        }
      }
      // O^T += V^T P^T, two 32-key chunks; k-slot order: 4 keys of block 2c then 4 of 2c+1
#pragma unroll
      for (int c = 0; c < KT / 32; ++c) {
        Frag<T> pf[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          if constexpr (sizeof(T) == 2) {
            uint4 u;
            u.x = pack_bf16x2(s[2 * c][qs][0], s[2 * c][qs][1]);
            u.y = pack_bf16x2(s[2 * c][qs][2], s[2 * c][qs][3]);
            u.z = pack_bf16x2(s[2 * c + 1][qs][0], s[2 * c + 1][qs][1]);
            u.w = pack_bf16x2(s[2 * c + 1][qs][2], s[2 * c + 1][qs][3]);
            pf[qs].v[0] = u;
          } else {
            pf[qs].v[0] = make_uint4(__float_as_uint(s[2 * c][qs][0]), __float_as_uint(s[2 * c][qs][1]),
                                     __float_as_uint(s[2 * c][qs][2]), __float_as_uint(s[2 * c][qs][3]));
            pf[qs].v[sizeof(T) / 2 - 1] =
                make_uint4(__float_as_uint(s[2 * c + 1][qs][0]), __float_as_uint(s[2 * c + 1][qs][1]),
                           __float_as_uint(s[2 * c + 1][qs][2]), __float_as_uint(s[2 * c + 1][qs][3]));
          }
        }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          Frag<T> vf;
          if constexpr (BF) {
            // V^T rows ds*16 + lc, k-slots 0..3 = keys 32c + 4lg + 0..3 and
            // 4..7 = keys 32c + 16 + 4lg + 0..3: lane lc of each 16-lane group
            // addresses key row 32c + 4lg + (lc >> 2), columns ds*16 + 4(lc & 3)
            constexpr int LDV = VK ? KLD : VLD;
            const T* vsrc = (VK ? Kb : Vb) + (32 * c + 4 * lg + (lc >> 2)) * LDV + ds * 16 + 4 * (lc & 3);
            const uint2 lo = lds_read_tr16(vsrc);
            const uint2 hi = lds_read_tr16(vsrc + 16 * LDV);
            vf.v[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          } else {
            const T* vrow = Vb + (ds * 16 + lc) * VLD + 32 * c + lg * 4;
            vf.v[0] = *reinterpret_cast<const uint4*>(vrow);
            vf.v[sizeof(T) / 2 - 1] = *reinterpret_cast<const uint4*>(vrow + 16);
          }
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) mma(oacc[ds][qs], vf, pf[qs]);
        }
      }
    }
  };
  // Absorbed MLA queries: q_lat^T = Wuk[h]^T q_nope^T on the MFMA (k = nope,
  // in order, as a GEMM of the same operands), rounded to bf16 and staged with
  // RoPE(q_pe) in this wave's rows of the K buffers (free until the first K
  // tile is stored), then read back as the query fragments. Runs while the
  // first K tile's loads are in flight; every wave takes part (barriers).
  auto build_q = [&]() {
    static_assert(!VK || (DQK == DV + 32 && NW * QW <= 2 * KT), "absorbed MLA: 32 rope dims, staging fits Ks");
    if constexpr (VK) {
      T* Qs = &Ks[0][0] + wave * QW * KLD;
      const T* qn = reinterpret_cast<const T*>(a.qn);
      const T* wk = reinterpret_cast<const T*>(a.wukT) + (long long)h * DV * a.nope;
      constexpr int CB = DV / 16;
      f32x4 qa[CB][QS];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) qa[cb][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < a.nope; k0 += 32) {
        const int kk = k0 + lg * 8;
        const bool kin = kk < a.nope;  // nope is a multiple of 8: a lane's 8 k values are all in or all out
        Frag<T> bq[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const int qq = qs * 16 + lc;
          bq[qs] = (qq < nq && kin)
                       ? frag_lds<T>(qn + (long long)(qfirst + qq) * a.qn_ld + (long long)h * a.qn_hs + kk)
                       : frag_zero<T>();
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const Frag<T> wf = kin ? frag_lds<T>(wk + (long long)(cb * 16 + lc) * a.nope + kk) : frag_zero<T>();
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) mma(qa[cb][qs], wf, bq[qs]);
        }
      }
      // lane (lg, lc) holds q_lat[query qs*16 + lc][c = cb*16 + 4lg + 0..3]
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        T* qrow = Qs + (qs * 16 + lc) * KLD;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          *reinterpret_cast<uint2*>(qrow + cb * 16 + 4 * lg) =
              make_uint2(pack_bf16x2(qa[cb][qs][0], qa[cb][qs][1]), pack_bf16x2(qa[cb][qs][2], qa[cb][qs][3]));
        // RoPE pairs (j, j + 16), j = 4lg .. 4lg + 3, of the 32 rope dims
        const int qq = qs * 16 + lc;
        uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
        if (qq < nq) {
          const T* src = qn + (long long)(qfirst + qq) * a.qn_ld + (long long)h * a.qn_hs + a.nope;
          const uint2 u1 = *reinterpret_cast<const uint2*>(src + 4 * lg);
          const uint2 u2 = *reinterpret_cast<const uint2*>(src + 16 + 4 * lg);
          const float4 c4 = *reinterpret_cast<const float4*>(a.cosb + qpos[qs] * 16 + 4 * lg);
          const float4 s4 = *reinterpret_cast<const float4*>(a.sinb + qpos[qs] * 16 + 4 * lg);
          const float x1[4] = {__uint_as_float(u1.x << 16), __uint_as_float(u1.x & 0xffff0000u),
                               __uint_as_float(u1.y << 16), __uint_as_float(u1.y & 0xffff0000u)};
          const float x2[4] = {__uint_as_float(u2.x << 16), __uint_as_float(u2.x & 0xffff0000u),
                               __uint_as_float(u2.y << 16), __uint_as_float(u2.y & 0xffff0000u)};
          const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
          float y1[4], y2[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {  // explicit roundings: the same in every instantiation
            y1[r] = __fmaf_rn(x1[r], cs[r], -(x2[r] * sn[r]));
            y2[r] = __fmaf_rn(x1[r], sn[r], x2[r] * cs[r]);
          }
          lo = make_uint2(pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]));
          hi = make_uint2(pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]));
        }
        *reinterpret_cast<uint2*>(qrow + DV + 4 * lg) = lo;
        *reinterpret_cast<uint2*>(qrow + DV + 16 + 4 * lg) = hi;
      }
      __syncthreads();
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[qs][ks] = frag_lds<T>(Qs + (qs * 16 + lc) * KLD + ks * 32 + lg * 8);
      __syncthreads();  // every wave holds its queries before the K tiles overwrite the staging
    }
  };
  if constexpr (QW == 16) {
    // tile kt sits in LDS buffer kt & 1; register set (kt & 1) receives tile
    // kt + 2 while tile kt is multiplied, and tile kt + 1 (in the other set,
    // loaded one tile earlier) is written to the other LDS buffer afterwards
    if (kt_begin < nkt) gload(kt_begin * KT, rk0, rv0);
    if (kt_begin + 1 < nkt) gload((kt_begin + 1) * KT, rk1, rv1);
    build_q();
    if (kt_begin < nkt) sstore(0, rk0, rv0);
    __syncthreads();
    for (int kt = kt_begin; kt < nkt; kt += 2) {
      if (kt + 2 < nkt) gload((kt + 2) * KT, rk0, rv0);
      tile(kt, 0);
      if (kt + 1 < nkt) sstore(1, rk1, rv1);
      __syncthreads();
      if (kt + 1 >= nkt) break;
      if (kt + 3 < nkt) gload((kt + 3) * KT, rk1, rv1);
      tile(kt + 1, 1);
      if (kt + 2 < nkt) sstore(0, rk0, rv0);
      __syncthreads();
    }
  } else {
    // wide query slices keep one tile in flight (fewer registers, more
    // workgroups per CU)
    if (kt_begin < nkt) gload(kt_begin * KT, rk0, rv0);
    build_q();
    if (kt_begin < nkt) sstore(0, rk0, rv0);
    __syncthreads();
    for (int kt = kt_begin; kt < nkt; ++kt) {
      const int buf = (kt - kt_begin) & 1;
      if (kt + 1 < nkt) gload((kt + 1) * KT, rk0, rv0);
      tile(kt, buf);
      if (kt + 1 < nkt) sstore(buf ^ 1, rk0, rv0);
      __syncthreads();
    }
  }

  if (split) {
    // Partial result of this key range, unnormalised. The ranges of one
    // (sequence, head group) may run on different XCDs (separate L2s), so the
    // partials are written and read with device-coherent accesses (agent-scope
    // atomic stores and loads) and counted with a device atomic; the range
    // that finishes last forms o.
    constexpr int SC = __HIP_MEMORY_SCOPE_AGENT;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int qq = qs * 16 + lc;
      if (qq >= nq) continue;
      const long long pr = ((long long)outer * a.B + (qfirst + qq)) * a.H + h;
      if (lg == 0) {
        __hip_atomic_store(a.part_m + pr, mrow[qs], __ATOMIC_RELAXED, SC);
        __hip_atomic_store(a.part_l + pr, lrow[qs], __ATOMIC_RELAXED, SC);
      }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __hip_atomic_store(a.part_o + pr * DV + ds * 16 + lg * 4 + r, oacc[ds][qs][r], __ATOMIC_RELAXED, SC);
    }
    __shared__ int s_last;
    // Release: every thread's partial stores happen before the count that
    // publishes them (an agent-scope release fence in each thread, then the
    // workgroup barrier, then one relaxed increment). Acquire in the range
    // that counts last, before it reads the other ranges' partials.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    const int grp = (int)(blockIdx.x % bz);             // (sequence b, head group)
    if (tid == 0) s_last = __hip_atomic_fetch_add(a.split_cnt + grp, 1, __ATOMIC_RELAXED, SC) == a.nsplit - 1;
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) __hip_atomic_store(a.split_cnt + grp, 0, __ATOMIC_RELAXED, SC);  // ready for the next launch
    // merge: one wave per head of the group, lane l owns columns 2l, 2l+1 of
    // the sequence's query row (row b: one query per sequence in decode)
    if (wave >= NHB) return;
    const int hh = (int)(blockIdx.x % nhg) * NHB + wave;
    const long long i = b;
    float M = -INFINITY;
    for (int r = 0; r < a.nsplit; ++r)
      M = fmaxf(M, __hip_atomic_load(a.part_m + ((long long)r * a.B + i) * a.H + hh, __ATOMIC_RELAXED, SC));
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    const int d = 2 * lane;
    for (int r = 0; r < a.nsplit; ++r) {
      const long long pr = ((long long)r * a.B + i) * a.H + hh;
      const float m = __hip_atomic_load(a.part_m + pr, __ATOMIC_RELAXED, SC);
      if (m == -INFINITY) continue;                 // an empty key range
      const float wgt = exp2f(m - M);
      L += wgt * __hip_atomic_load(a.part_l + pr, __ATOMIC_RELAXED, SC);
      if (d < DV) {
        o0 += wgt * __hip_atomic_load(a.part_o + pr * DV + d, __ATOMIC_RELAXED, SC);
        o1 += wgt * __hip_atomic_load(a.part_o + pr * DV + d + 1, __ATOMIC_RELAXED, SC);
      }
    }
    if (d < DV) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      T* Om = reinterpret_cast<T*>(a.o) + i * a.o_ld + (long long)hh * a.o_hs + d;
      Om[0] = ST<T>::from_f(o0 * inv);
      Om[1] = ST<T>::from_f(o1 * inv);
    }
    return;
  }
  if constexpr (VK) {
    // value up-projection o = o_lat Wuv[h]^T on the MFMA, o_lat normalised and
    // rounded to bf16 as a stored o_lat would be. The accumulators hold o_lat
    // transposed, so a lane's 8 k-slots of k-step ks are c = 32ks + 4lg + 0..3
    // and 32ks + 16 + 4lg + 0..3 (the layout of P above); the Wuv fragments
    // are read in the same order.
    constexpr int KC = DV / 32;
    Frag<T> of[KC][QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const float inv = lrow[qs] > 0.f ? 1.f / lrow[qs] : 0.f;
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        const f32x4& p0 = oacc[2 * ks][qs];
        const f32x4& p1 = oacc[2 * ks + 1][qs];
        of[ks][qs].v[0] = make_uint4(pack_bf16x2(p0[0] * inv, p0[1] * inv), pack_bf16x2(p0[2] * inv, p0[3] * inv),
                                     pack_bf16x2(p1[0] * inv, p1[1] * inv), pack_bf16x2(p1[2] * inv, p1[3] * inv));
      }
    }
    const T* wv = reinterpret_cast<const T*>(a.wuv) + (long long)h * a.vd * DV;
    T* Ov = reinterpret_cast<T*>(a.ov);
    for (int j0 = 0; j0 < a.vd; j0 += 16) {
      const int j = j0 + lc;
      f32x4 acc[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) acc[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        Frag<T> wf = frag_zero<T>();
        if (j < a.vd) {
          const T* p = wv + (long long)j * DV + 32 * ks + 4 * lg;
          const uint2 lo = *reinterpret_cast<const uint2*>(p), hi = *reinterpret_cast<const uint2*>(p + 16);
          wf.v[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) mma(acc[qs], wf, of[ks][qs]);
      }
      // lane (lg, lc): output columns j0 + 4lg + 0..3 of query qs*16 + lc
      const int jr = j0 + 4 * lg;
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const int qq = qs * 16 + lc;
        if (qq >= nq || jr >= a.vd) continue;
        float v[4] = {acc[qs][0], acc[qs][1], acc[qs][2], acc[qs][3]};
        store4<T>(Ov + (long long)(qfirst + qq) * a.ov_ld + (long long)h * a.vd + jr, v);
      }
    }
    return;
  }
  T* O = reinterpret_cast<T*>(a.o);
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qq = qs * 16 + lc;
    if (qq >= nq) continue;
    const int i = qfirst + qq;
    const float inv = lrow[qs] > 0.f ? 1.f / lrow[qs] : 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      float v[4] = {oacc[ds][qs][0] * inv, oacc[ds][qs][1] * inv, oacc[ds][qs][2] * inv,
                    oacc[ds][qs][3] * inv};
      store4<T>(O + (long long)i * a.o_ld + (long long)h * a.o_hs + ds * 16 + lg * 4, v);
    }
  }
}

template <typename T, int DQK, int DV, int QW, int NHB, bool VK, int NW = 4>
static hipError_t attn_launch(const AttnArgs& a, hipStream_t s) {
  // 128-key tiles for bf16 heads up to 64 wide (measured faster on the gqa and
  // ACT workloads); 64-key tiles otherwise (LDS and registers)
  constexpr int KT = (sizeof(T) == 2 && DQK <= 64) ? 128 : 64;
  constexpr int BQ = QW * (NW / NHB);
  dim3 grid((a.dec ? (a.nsplit > 1 ? a.nsplit : 1) : (a.S + BQ - 1) / BQ) * a.B * (a.H / NHB));
  hipLaunchKernelGGL((k_attention<T, DQK, DV, QW, NHB, KT, NW, VK>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

// Heads per workgroup: up to 4 heads that share a kv head; 16-row query slices
// (32 rows when the launch has blocks to spare: every key and value fragment
// read from LDS then feeds two MFMAs; measured in place, MLA forward -7 %,
// wide_moe -4 %).
template <typename T, int DQK, int DV, bool VK>
static hipError_t attn_pick(const AttnArgs& a, hipStream_t s) {
  const int G = a.H / a.KV;
  const int nhb = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const long long blocks16 = (long long)(a.dec ? 1 : (a.S + 63) / 64) * a.B * a.H;  // 64 rows per block per head
  const bool wide = blocks16 * 2 >= 1024 && !a.narrow;
  if (nhb == 4) return wide ? attn_launch<T, DQK, DV, 32, 4, VK>(a, s) : attn_launch<T, DQK, DV, 16, 4, VK>(a, s);
  if (nhb == 2) return wide ? attn_launch<T, DQK, DV, 32, 2, VK>(a, s) : attn_launch<T, DQK, DV, 16, 2, VK>(a, s);
  return wide ? attn_launch<T, DQK, DV, 32, 1, VK>(a, s) : attn_launch<T, DQK, DV, 16, 1, VK>(a, s);
}

template <typename T>
static hipError_t attn_dispatch(const AttnArgs& a, hipStream_t s) {
  const int dq = a.dqk, dv = a.dv;
  // bf16 absorbed MLA: the value is the prefix of the key row; its V^T
  // fragments are read from the K tile
  const bool vk = sizeof(T) == 2 && a.v == a.k && a.v_ld == a.k_ld && a.v_hs == a.k_hs && dv <= dq;
  const bool split = a.dec && a.nsplit > 1;
  if (vk && (!a.qn || !a.wukT || !a.cosb || !a.sinb || a.nope <= 0 || a.nope % 8 ||
             (!split && (!a.wuv || !a.ov || a.vd <= 0 || a.vd % 8))))
    return hipErrorInvalidValue;
  if (dq == 16 && dv == 16) return attn_pick<T, 16, 16, false>(a, s);
  if (dq == 32 && dv == 32) return attn_pick<T, 32, 32, false>(a, s);
  if (dq == 64 && dv == 64) return attn_pick<T, 64, 64, false>(a, s);
  if (dq == 128 && dv == 128) return attn_pick<T, 128, 128, false>(a, s);
  if (dq == 160 && dv == 128)
    return vk ? attn_pick<T, 160, 128, sizeof(T) == 2>(a, s) : attn_pick<T, 160, 128, false>(a, s);
  if (dq == 96 && dv == 64)
    return vk ? attn_pick<T, 96, 64, sizeof(T) == 2>(a, s) : attn_pick<T, 96, 64, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.H % a.KV) return hipErrorInvalidValue;
  if (a.dec && a.nsplit > 1 && (!a.part_o || !a.part_m || !a.part_l || !a.split_cnt || a.rows || a.seg || a.dv > 128))
    return hipErrorInvalidValue;
  return a.dtype == DT_F32 ? attn_dispatch<float>(a, s) : attn_dispatch<bf16_t>(a, s);
}

}  // namespace rdt
