// CoWindow Attention backward, bf16, head dim 128, for gfx950.
//
// Gradients of the same masked softmax attention the forward computes (the pages state
// that the pattern supports training forward and backward — beyondmarketintelligence.com
// post, second paragraph; "CoWindow Attention" abstract), recomputed from the saved
// logsumexp:
//   P = exp(scale q.k - LSE), Delta_i = dO_i . O_i, dP = dO V^T, dS = P (dP - Delta)
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
// Three kernels, no atomics (deterministic):
//   delta  : Delta per (row, query head);
//   dq     : one work item per (KV head, q-block of 128 / G tokens), walking the row list
//            of visible 128-key blocks: S^T, dP^T, dS^T on MFMA, dQ^T += K^T dS^T with
//            K^T read by ds_read_b64_tr_b16 from the row-major LDS tile;
//   dkdv   : one work item per (KV head, 128-key block), walking the column list of
//            visible q-blocks; each of the 4 waves keeps 32 keys of K and V in registers
//            and accumulates dK, dV for them over all G query heads of the KV head:
//            S = Q K^T and dP = dO V^T on MFMA, then dV += P^T dO and dK += dS^T Q with
//            P, dS taken from the accumulator registers as A operands (each as a bf16
//            hi + lo pair) and dO, Q read transposed from LDS.
// Rows of a q-block are token-major (row r = token * G + head-in-group); rows beyond
// G * Bq or Lq carry LSE = +inf and Delta = 0 so that they contribute nothing.

#include "cowa.h"
#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int ROWS = kBwdRows;  // 128 query rows per q-block
constexpr int BK = kBwdBk;      // 128 keys per k-block
constexpr int SUB = 64;         // keys staged per LDS sub-tile in the dq kernel

// x -> (hi, lo) with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits as two
// bf16 MFMA operands.  Done for 8 values at once with packed conversions; hi is widened
// back to fp32 exactly by bit shifts.
__device__ __forceinline__ void split_hi_lo(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 wh, wl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 h = {(__bf16)x[2 * k], (__bf16)x[2 * k + 1]};
    const unsigned w = __builtin_bit_cast(unsigned, h);
    // (w << 16 as a byte permute: written as a shift, it gets re-derived from a second
    // conversion)
    const float h0 = __uint_as_float(__builtin_amdgcn_perm(w, w, 0x01000c0cu));
    const float h1 = __uint_as_float(w & 0xffff0000u);
    const bf16x2 l = {(__bf16)(x[2 * k] - h0), (__bf16)(x[2 * k + 1] - h1)};
    wh[k] = w;
    wl[k] = __builtin_bit_cast(unsigned, l);
  }
  hi = __builtin_bit_cast(bf16x8, wh);
  lo = __builtin_bit_cast(bf16x8, wl);
}

// ------------------------------------------------------------------------ Delta
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, hq) flat
  const int li = threadIdx.x & 15;
  const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 ow = *(const u32x4*)((const __bf16*)a.o + row * D + 8 * li);
    const u32x4 dw = *(const u32x4*)((const __bf16*)a.dout + row * D + 8 * li);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(ow[k] << 16), __uint_as_float(dw[k] << 16), acc);
      acc = fmaf(__uint_as_float(ow[k] & 0xffff0000u), __uint_as_float(dw[k] & 0xffff0000u), acc);
    }
  }
  acc += __shfl_xor(acc, 1, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 8, 16);
  if (row < nrows && li == 0) {
    const int hq = (int)(row % a.Hq);
    const int64_t bt = row / a.Hq;
    const int t = (int)(bt % a.Lq);
    const int b = (int)(bt / a.Lq);
    a.delta[((int64_t)b * a.Hq + hq) * a.Lq + t] = acc;
  }
}

// ------------------------------------------------------------------------ dQ
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 sK[SUB * D];  // swizzled rows (lds_swz)
  __shared__ __attribute__((aligned(16))) __bf16 sV[SUB * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = a.row_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const __bf16* dO = (const __bf16*)a.dout;

  // this lane's query row (column of the transposed products)
  const int r = wave * 32 + n;
  const int rt = r / G;
  const int t = qb * Bq + rt;
  const int hq = h * G + (r - rt * G);
  const bool rvalid = (rt < Bq) && (t < a.Lq);
  const int p = t + off;
  float lse2 = INFINITY, dlt = 0.f;
  bf16x8 qf[8], df[8];
  if (rvalid) {
    lse2 = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + t] * kLog2e;
    dlt = a.delta[((int64_t)b * a.Hq + hq) * a.Lq + t];
    const int64_t ro = (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 8 * h2;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      qf[dd] = load16(Q + ro + 16 * dd);
      df[dd] = load16(dO + ro + 16 * dd);
    }
  } else {
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) qf[dd] = df[dd] = zero_bf16x8();
  }
  if (lse2 == -INFINITY) lse2 = INFINITY;  // a row with no visible key has P = 0

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);

  // staging of one 64-key sub-tile: chunks tid + 256 u (u < 4), row id / 16, col id % 16
  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  const int n_sub = 2 * (e1 - e0);
  u32x4 pk[4], pv[4];
  auto fetch = [&](int sidx) {
    const int kb = a.row_ent[e0 + (sidx >> 1)] >> 1;
    const int jb = kb * BK + (sidx & 1) * SUB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      const int j = jb + row;
      if (j < a.Lk) {
        const int64_t o = (((int64_t)b * a.Lk + j) * a.Hkv + h) * D + 8 * cc;
        pk[u] = *(const u32x4*)(K + o);
        pv[u] = *(const u32x4*)(V + o);
      } else {
        pk[u] = u32x4{0, 0, 0, 0};
        pv[u] = u32x4{0, 0, 0, 0};
      }
    }
  };
  if (n_sub > 0) fetch(0);

  for (int sidx = 0; sidx < n_sub; ++sidx) {
    const int ent = a.row_ent[e0 + (sidx >> 1)];
    const int jb = (ent >> 1) * BK + (sidx & 1) * SUB;
    const bool partial = ent & 1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      *(u32x4*)(sK + lds_swz(row, 8 * cc)) = pk[u];
      *(u32x4*)(sV + lds_swz(row, 8 * cc)) = pv[u];
    }
    __syncthreads();
    if (sidx + 1 < n_sub) fetch(sidx + 1);

    // S^T and dP^T for both 32-key halves first: four independent accumulation chains
    f32x16 s2[SUB / 32], dp2[SUB / 32];
#pragma unroll
    for (int k2 = 0; k2 < SUB / 32; ++k2)
#pragma unroll
      for (int i = 0; i < 16; ++i) s2[k2][i] = dp2[k2][i] = 0.f;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd)
#pragma unroll
      for (int k2 = 0; k2 < SUB / 32; ++k2) {
        const bf16x8 kf = load16(sK + lds_swz(32 * k2 + n, 16 * dd + 8 * h2));
        const bf16x8 vf = load16(sV + lds_swz(32 * k2 + n, 16 * dd + 8 * h2));
        s2[k2] = mfma32x32x16(kf, qf[dd], s2[k2]);
        dp2[k2] = mfma32x32x16(vf, df[dd], dp2[k2]);
      }
#pragma unroll
    for (int k2 = 0; k2 < SUB / 32; ++k2) {
      const f32x16& s = s2[k2];
      const f32x16& dp = dp2[k2];
      float pr[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -lse2));
      if (partial) {  // one uniform branch; the predicate per element, branch-free
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = jb + 32 * k2 + 8 * (i >> 2) + 4 * h2 + (i & 3);
          pr[i] = (rvalid & visible(p, j, a.Lk, a.win.sink, a.win.near_w, band)) ? pr[i] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = pr[i] * (dp[i] - dlt);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 dsf = join(to_bf16x4(ds[8 * hf], ds[8 * hf + 1], ds[8 * hf + 2], ds[8 * hf + 3]),
                                to_bf16x4(ds[8 * hf + 4], ds[8 * hf + 5], ds[8 * hf + 6], ds[8 * hf + 7]));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int r0 = 32 * k2 + 16 * hf + vrow, col = 32 * db + vcol;
          const bf16x8 ktf = join(lds_read_tr4(sK + lds_swz(r0, col)), lds_read_tr4(sK + lds_swz(r0 + 8, col)));
          acc[db] = mfma32x32x16(ktf, dsf, acc[db]);
        }
      }
    }
  }

  if (rvalid) {
    __bf16* dq = (__bf16*)a.dq + (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 4 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const bf16x4 v = to_bf16x4(acc[db][4 * q4] * a.scale, acc[db][4 * q4 + 1] * a.scale,
                                   acc[db][4 * q4 + 2] * a.scale, acc[db][4 * q4 + 3] * a.scale);
        *(u32x2*)(dq + 32 * db + 8 * q4) = __builtin_bit_cast(u32x2, v);
      }
  }
}

// ------------------------------------------------------------------------ dK, dV
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 sQ[ROWS * D];  // swizzled rows (lds_swz)
  __shared__ __attribute__((aligned(16))) __bf16 sD[ROWS * D];
  __shared__ __attribute__((aligned(16))) float sL[ROWS];
  __shared__ __attribute__((aligned(16))) float sT[ROWS];
  __shared__ int sTok[ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = a.col_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nkb;
  const int kb = item - h * a.nkb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const __bf16* dO = (const __bf16*)a.dout;

  // this lane's key (column of S and dP)
  const int j = kb * BK + wave * 32 + n;
  const bool kvalid = j < a.Lk;
  bf16x8 kf[8], vf[8];
  {
    const int64_t ko = (((int64_t)b * a.Lk + (kvalid ? j : 0)) * a.Hkv + h) * D + 8 * h2;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      kf[dd] = kvalid ? load16(K + ko + 16 * dd) : zero_bf16x8();
      vf[dd] = kvalid ? load16(V + ko + 16 * dd) : zero_bf16x8();
    }
  }

  f32x16 accK[4], accV[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) accK[db][i] = accV[db][i] = 0.f;

  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);

  const int e0 = a.col_ptr[item], e1 = a.col_ptr[item + 1];
  // staging of one q-block: Q and dO rows, chunks tid + 256 u (u < 8), row id / 16
  u32x4 pq[8], pd[8];
  float plse = INFINITY, pdel = 0.f;
  int ptok = 0x40000000;
  auto fetch = [&](int e) {
    const int qb = a.col_ent[e] >> 1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      const int rt = row / G;
      const int t = qb * Bq + rt;
      if (rt < Bq && t < a.Lq) {
        const int64_t o = (((int64_t)b * a.Lq + t) * a.Hq + h * G + (row - rt * G)) * D + 8 * cc;
        pq[u] = *(const u32x4*)(Q + o);
        pd[u] = *(const u32x4*)(dO + o);
      } else {
        pq[u] = u32x4{0, 0, 0, 0};
        pd[u] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < ROWS) {
      const int rt = tid / G;
      const int t = qb * Bq + rt;
      plse = INFINITY;
      pdel = 0.f;
      ptok = 0x40000000;
      if (rt < Bq && t < a.Lq) {
        const int64_t si = ((int64_t)b * a.Hq + h * G + (tid - rt * G)) * a.Lq + t;
        const float lv = a.lse[si];
        plse = lv == -INFINITY ? INFINITY : lv * kLog2e;
        pdel = a.delta[si];
        ptok = t;
      }
    }
  };
  if (e0 < e1) fetch(e0);

  for (int e = e0; e < e1; ++e) {
    const bool partial = a.col_ent[e] & 1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      *(u32x4*)(sQ + lds_swz(row, 8 * cc)) = pq[u];
      *(u32x4*)(sD + lds_swz(row, 8 * cc)) = pd[u];
    }
    if (tid < ROWS) {
      sL[tid] = plse;
      sT[tid] = pdel;
      sTok[tid] = ptok;
    }
    __syncthreads();
    if (e + 1 < e1) fetch(e + 1);

#pragma unroll
    for (int rb = 0; rb < ROWS / 32; ++rb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const bf16x8 qa = load16(sQ + lds_swz(32 * rb + n, 16 * dd + 8 * h2));
        const bf16x8 da = load16(sD + lds_swz(32 * rb + n, 16 * dd + 8 * h2));
        s = mfma32x32x16(qa, kf[dd], s);
        dp = mfma32x32x16(da, vf[dd], dp);
      }
      // element i: row 32 rb + 8 (i / 4) + 4 h2 + i % 4, key j
      float pr[16], ds[16];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int rr = 32 * rb + 8 * i4 + 4 * h2;
        const f32x4 l4 = *(const f32x4*)(sL + rr);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[4 * i4 + i] = __builtin_amdgcn_exp2f(fmaf(s[4 * i4 + i], a.scale_log2, -l4[i]));
      }
      if (partial) {  // one uniform branch; the predicate per element, branch-free
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int rr = 32 * rb + 8 * i4 + 4 * h2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool vis = kvalid & visible(sTok[rr + i] + off, j, a.Lk, a.win.sink, a.win.near_w, band);
            pr[4 * i4 + i] = vis ? pr[4 * i4 + i] : 0.f;
          }
        }
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 t4 = *(const f32x4*)(sT + 32 * rb + 8 * i4 + 4 * h2);
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[4 * i4 + i] = pr[4 * i4 + i] * (dp[4 * i4 + i] - t4[i]);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // P and dS as bf16 pairs hi + lo (~16 mantissa bits): dV and dK sum them over many
        // rows with strong cancellation, so a single bf16 rounding would dominate the error
        bf16x8 pa, pl, sa, sl;
        split_hi_lo(pr + 8 * hf, pa, pl);
        split_hi_lo(ds + 8 * hf, sa, sl);
        // hi products for all 4 column blocks, then the lo ones: an accumulator is next
        // updated only after 7 independent MFMAs
        bf16x8 dt[4], qt[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int r0 = 32 * rb + 16 * hf + vrow, col = 32 * db + vcol;
          dt[db] = join(lds_read_tr4(sD + lds_swz(r0, col)), lds_read_tr4(sD + lds_swz(r0 + 8, col)));
          qt[db] = join(lds_read_tr4(sQ + lds_swz(r0, col)), lds_read_tr4(sQ + lds_swz(r0 + 8, col)));
          accV[db] = mfma32x32x16(pa, dt[db], accV[db]);
          accK[db] = mfma32x32x16(sa, qt[db], accK[db]);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          accV[db] = mfma32x32x16(pl, dt[db], accV[db]);
          accK[db] = mfma32x32x16(sl, qt[db], accK[db]);
        }
      }
    }
  }

  // element i of accK[db] / accV[db]: key 32 wave + 8 (i / 4) + 4 h2 + i % 4, dim 32 db + n
  __bf16* dK = (__bf16*)a.dk;
  __bf16* dV = (__bf16*)a.dv;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int jj = kb * BK + wave * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
      if (jj < a.Lk) {
        const int64_t o = (((int64_t)b * a.Lk + jj) * a.Hkv + h) * D + 32 * db + n;
        dK[o] = (__bf16)(accK[db][i] * a.scale);
        dV[o] = (__bf16)accV[db][i];
      }
    }
}

}  // namespace

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, int stages, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (stages & COWA_BWD_DELTA) {
    const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((nrows + 15) / 16)), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (stages & COWA_BWD_DQ) {
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(a.Hkv * a.nqb, a.B), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (stages & COWA_BWD_DKDV) {
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(a.Hkv * a.nkb, a.B), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return err;
}

}  // namespace cowa
