// Backward kernels: recompute the probability tiles from the saved
// log-sum-exp instead of storing them ("Flash Attention, From First
// Principles", "The backward pass -- resurrection"; "FlashAttention from
// scratch", Step 4 and Follow-up questions).
//
// Three launches on the caller's stream:
//   1. bwd_pre:   D_i = sum_c dO_ic * O_ic (fp32) and zero the fp32 dQ
//                 accumulator.
//   2. bwd_main:  one workgroup per 128-key tile of one (batch, head); each of
//                 the 4 waves owns 32 keys and keeps K, V (as MFMA operands)
//                 and its dK, dV accumulators in registers for the whole
//                 kernel.  Query blocks stream past the resident key tile; per
//                 block a wave recomputes
//                   S  = Q K^T                 (MFMA, lane = key)
//                   P  = exp(scale*S - L)      (L = saved lse; masked -> 0)
//                   dV^T += dO^T P             (MFMA)
//                   dP = dO V^T                (MFMA)
//                   dS = P * (dP - D)
//                   dK^T += Q^T dS             (MFMA)
//                 then dS goes through LDS so that each wave can form one
//                 32x32 block of dQ = dS K over all 128 keys (MFMA, K^T kept
//                 in LDS) and add it, times scale, into the fp32 accumulator
//                 with hardware float atomics.  Query blocks wholly before the
//                 key tile are skipped under causal masking ("LLM Architecture
//                 Refresh [3]", section 7).
//   3. bwd_dq:    dQ = bf16(accumulator).
//
// The P and dS registers of the S / dP accumulators are already in the
// B-operand layout for dV^T and dK^T (keys across lanes, queries across
// registers); the matching A operands (dO^T, Q^T) are stored transposed in
// LDS in the same query order, exactly as V^T in the forward.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBKN = 128;  // keys per workgroup (4 waves x 32)

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero the dQ accumulator
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dv,
                                                      float* __restrict__ dQacc, size_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 features each
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = row * D + part * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_bits_to_float(a[i] & 0xffffu) * bf16_bits_to_float(b[i] & 0xffffu);
      acc += bf16_bits_to_float(a[i] >> 16) * bf16_bits_to_float(b[i] >> 16);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQacc + off) = z;
    *reinterpret_cast<f32x4*>(dQacc + off + 4) = z;
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && part == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// 3. dQ accumulator -> bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ dQacc,
                                                     uint16_t* __restrict__ dQ, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(dQacc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(dQacc + 8 * i + 4);
  u32x4 out = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
               pack_bf16x2(b[2], b[3])};
  *reinterpret_cast<u32x4*>(dQ + 8 * i) = out;
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int BQ = D == 128 ? 32 : 64;   // queries per streamed block
  static constexpr int NQS = BQ / 32;             // 32-query sub-blocks
  static constexpr int RS = D + 8;                // Q / dO row stride (elements)
  static constexpr int TS = BQ + 8;               // Q^T / dO^T row stride
  static constexpr int KTS = kBKN + 8;            // K^T row stride
  static constexpr int DSS = kBKN + 8;            // dS row stride
  static constexpr int NDC = D / 16;              // 16-feature chunks
  static constexpr int NDB = D / 32;              // 32-feature blocks
  // LDS layout (bf16 elements)
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_Q = OFF_KT + D * KTS;
  static constexpr int OFF_QT = OFF_Q + BQ * RS;
  static constexpr int OFF_DO = OFF_QT + D * TS;
  static constexpr int OFF_DOT = OFF_DO + BQ * RS;
  static constexpr int OFF_DS = OFF_DOT + D * TS;
  static constexpr int OFF_STAT = OFF_DS + BQ * DSS;   // 2*BQ floats (lse2, D)
  static constexpr int SMEM_BYTES = OFF_STAT * 2 + 2 * BQ * 4;
  // 4x4 blocks of one [BQ, D] tile per thread
  static constexpr int BLK = (BQ / 4) * (D / 4) / 256;
  static_assert(BLK * 256 * 16 == BQ * D, "query tile split");
  // waves for dQ: one 32x32 block of [BQ, D] each
  static_assert(NQS * NDB == 4, "dQ blocks per workgroup");
  static constexpr int KT_BLK = (kBKN / 4) * (D / 4) / 256;
};

template <int D>
struct QRegs {
  u32x2 q[BwdCfg<D>::BLK][4];
  u32x2 g[BwdCfg<D>::BLK][4];   // dO
  float lse2, dv;
};

template <int D>
__device__ __forceinline__ void load_qblock(QRegs<D>& r, const uint16_t* __restrict__ Qh,
                                            const uint16_t* __restrict__ dOh,
                                            const float* __restrict__ lseh,
                                            const float* __restrict__ Dh, int q0, int N,
                                            int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::BLK; ++i) {
    const int bi = i * 256 + tid;
    const int qg = bi % (C::BQ / 4);
    const int dg = bi / (C::BQ / 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int qrow = q0 + 4 * qg + rr;
      if (qrow < N) {
        r.q[i][rr] = *reinterpret_cast<const u32x2*>(Qh + (size_t)qrow * D + 4 * dg);
        r.g[i][rr] = *reinterpret_cast<const u32x2*>(dOh + (size_t)qrow * D + 4 * dg);
      } else {
        r.q[i][rr] = u32x2{0u, 0u};
        r.g[i][rr] = u32x2{0u, 0u};
      }
    }
  }
  r.lse2 = 0.f;
  r.dv = 0.f;
  if (tid < C::BQ && q0 + tid < N) {
    r.lse2 = lseh[q0 + tid] * kLog2e;
    r.dv = Dh[q0 + tid];
  }
}

// Writes one 4x4 block (rows 4g..4g+3, features 4dg..4dg+3) both row-major
// and transposed (rows permuted by tr_group_pos within 16-row chunks).
template <int RSTRIDE, int TSTRIDE>
__device__ __forceinline__ void store_4x4(const u32x2* v, uint16_t* rowmajor, uint16_t* trans,
                                          int g, int dg) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    *reinterpret_cast<u32x2*>(rowmajor + (4 * g + rr) * RSTRIDE + 4 * dg) = v[rr];
  const int pos = 16 * (g >> 2) + 4 * tr_group_pos(g & 3);
  uint16_t* base = trans + (4 * dg) * TSTRIDE + pos;
  *reinterpret_cast<u32x2*>(base + 0 * TSTRIDE) =
      u32x2{pack_lo16(v[0].x, v[1].x), pack_lo16(v[2].x, v[3].x)};
  *reinterpret_cast<u32x2*>(base + 1 * TSTRIDE) =
      u32x2{pack_hi16(v[0].x, v[1].x), pack_hi16(v[2].x, v[3].x)};
  *reinterpret_cast<u32x2*>(base + 2 * TSTRIDE) =
      u32x2{pack_lo16(v[0].y, v[1].y), pack_lo16(v[2].y, v[3].y)};
  *reinterpret_cast<u32x2*>(base + 3 * TSTRIDE) =
      u32x2{pack_hi16(v[0].y, v[1].y), pack_hi16(v[2].y, v[3].y)};
}

template <int D>
__device__ __forceinline__ void store_qblock(const QRegs<D>& r, uint16_t* smem, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::BLK; ++i) {
    const int bi = i * 256 + tid;
    const int qg = bi % (C::BQ / 4);
    const int dg = bi / (C::BQ / 4);
    store_4x4<C::RS, C::TS>(r.q[i], smem + C::OFF_Q, smem + C::OFF_QT, qg, dg);
    store_4x4<C::RS, C::TS>(r.g[i], smem + C::OFF_DO, smem + C::OFF_DOT, qg, dg);
  }
  float* stat = reinterpret_cast<float*>(smem + C::OFF_STAT);
  if (tid < C::BQ) {
    stat[tid] = r.lse2;
    stat[C::BQ + tid] = r.dv;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv, float* __restrict__ dQacc,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, int nkt, float scale,
    float c2) {
  using C = BwdCfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, kt;
  map_tile(blockIdx.x, BH, nkt, false, &bh, &kt);
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const uint16_t* dOh = dO + base;
  const float* lseh = LSE + (size_t)bh * N;
  const float* Dh = Dv + (size_t)bh * N;
  float* dQh = dQacc + base;

  const int k0 = kt * kBKN;
  const int wk0 = k0 + 32 * w;   // this wave's first key
  const int key = wk0 + n;       // this lane's key

  // K and V as B operands (lane = key, 8 consecutive features per chunk)
  bf16x8 kf[C::NDC], vf[C::NDC];
#pragma unroll
  for (int cc = 0; cc < C::NDC; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < N) {
      a = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + 16 * cc + 8 * h);
      b = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + 16 * cc + 8 * h);
    }
    kf[cc] = __builtin_bit_cast(bf16x8, a);
    vf[cc] = __builtin_bit_cast(bf16x8, b);
  }
  // K^T of the whole 128-key tile into LDS (natural key order) for dQ
#pragma unroll
  for (int i = 0; i < C::KT_BLK; ++i) {
    const int bi = i * 256 + tid;
    const int kg = bi % (kBKN / 4);
    const int dg = bi / (kBKN / 4);
    u32x2 v4[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kk = k0 + 4 * kg + rr;
      v4[rr] = kk < N ? *reinterpret_cast<const u32x2*>(Kh + (size_t)kk * D + 4 * dg)
                      : u32x2{0u, 0u};
    }
    uint16_t* tb = smem + C::OFF_KT + (4 * dg) * C::KTS + 4 * kg;
    *reinterpret_cast<u32x2*>(tb + 0 * C::KTS) =
        u32x2{pack_lo16(v4[0].x, v4[1].x), pack_lo16(v4[2].x, v4[3].x)};
    *reinterpret_cast<u32x2*>(tb + 1 * C::KTS) =
        u32x2{pack_hi16(v4[0].x, v4[1].x), pack_hi16(v4[2].x, v4[3].x)};
    *reinterpret_cast<u32x2*>(tb + 2 * C::KTS) =
        u32x2{pack_lo16(v4[0].y, v4[1].y), pack_lo16(v4[2].y, v4[3].y)};
    *reinterpret_cast<u32x2*>(tb + 3 * C::KTS) =
        u32x2{pack_hi16(v4[0].y, v4[1].y), pack_hi16(v4[2].y, v4[3].y)};
  }

  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  const int nqb = (N + C::BQ - 1) / C::BQ;
  const int qb0 = CAUSAL ? (k0 / C::BQ) : 0;

  QRegs<D> regs;
  if (qb0 < nqb) {
    load_qblock<D>(regs, Qh, dOh, lseh, Dh, qb0 * C::BQ, N, tid);
    store_qblock<D>(regs, smem, tid);
  }
  __syncthreads();

  const uint16_t* sQ = smem + C::OFF_Q;
  const uint16_t* sQT = smem + C::OFF_QT;
  const uint16_t* sDO = smem + C::OFF_DO;
  const uint16_t* sDOT = smem + C::OFF_DOT;
  uint16_t* sDS = smem + C::OFF_DS;
  const float* sStat = reinterpret_cast<const float*>(smem + C::OFF_STAT);

  for (int qb = qb0; qb < nqb; ++qb) {
    const int q0 = qb * C::BQ;
    const bool more = qb + 1 < nqb;
    if (more) load_qblock<D>(regs, Qh, dOh, lseh, Dh, q0 + C::BQ, N, tid);

    // the wave's keys are all after every query of the block: nothing to do
    const bool wave_dead = CAUSAL && (wk0 > q0 + C::BQ - 1);
#pragma unroll
    for (int qs = 0; qs < C::NQS; ++qs) {
      const int qs0 = q0 + 32 * qs;
      // a 32-query sub-block wholly before the wave's keys contributes nothing
      const bool sub_dead = wave_dead || (CAUSAL && wk0 > qs0 + 31);
      uint32_t pk[8], sk[8];
      if (!sub_dead) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const uint16_t* qrow = sQ + (32 * qs + n) * C::RS + 8 * h;
        const uint16_t* grow = sDO + (32 * qs + n) * C::RS + 8 * h;
#pragma unroll
        for (int cc = 0; cc < C::NDC; ++cc) {
          s = mfma_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(qrow + 16 * cc), kf[cc], s);
          dp = mfma_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(grow + 16 * cc), vf[cc], dp);
        }
        // registers r: query 32qs + 8(r/4) + 4h + r%4, key = this lane's key
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p2[2], ds2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ql = 32 * qs + 8 * ((r + u) >> 2) + 4 * h + ((r + u) & 3);
            const int qrow_g = q0 + ql;
            const float l2 = sStat[ql];
            const float dd = sStat[C::BQ + ql];
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + u], c2, -l2));
            bool dead = qrow_g >= N || key >= N;
            if (CAUSAL) dead = dead || key > qrow_g;
            p = dead ? 0.f : p;
            p2[u] = p;
            ds2[u] = p * (dp[r + u] - dd);
          }
          pk[r >> 1] = pack_bf16x2(p2[0], p2[1]);
          sk[r >> 1] = pack_bf16x2(ds2[0], ds2[1]);
        }
        // dV^T += dO^T P ; dK^T += Q^T dS   (k = queries of this sub-block)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 bp = __builtin_bit_cast(
              bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
          const bf16x8 bs = __builtin_bit_cast(
              bf16x8, u32x4{sk[4 * half], sk[4 * half + 1], sk[4 * half + 2], sk[4 * half + 3]});
          const int col = 32 * qs + 16 * half + 8 * h;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16x8 ag = *reinterpret_cast<const bf16x8*>(sDOT + (32 * db + n) * C::TS + col);
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQT + (32 * db + n) * C::TS + col);
            dv[db] = mfma_32x32x16_bf16(ag, bp, dv[db]);
            dk[db] = mfma_32x32x16_bf16(aq, bs, dk[db]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) sk[i] = 0u;
      }
      // dS (bf16) into LDS as [query][key of the 128-key tile]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qs + 8 * (r >> 2) + 4 * h + (r & 3);
        const uint16_t bits = (r & 1) ? (uint16_t)(sk[r >> 1] >> 16) : (uint16_t)(sk[r >> 1] & 0xffffu);
        sDS[ql * C::DSS + 32 * w + n] = bits;
      }
    }
    __syncthreads();

    // dQ block of this wave: queries 32*qsq.., features 32*dbq..
    {
      const int qsq = w / C::NDB;
      const int dbq = w % C::NDB;
      const int qs0 = q0 + 32 * qsq;
      // keys of the tile after every query of the sub-block contribute nothing
      int nkc = kBKN / 16;
      if (CAUSAL) {
        const int lim = qs0 + 31 - k0;
        nkc = lim < 0 ? 0 : min(kBKN / 16, lim / 16 + 1);
      }
      if (nkc > 0) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const uint16_t* arow = sDS + (32 * qsq + n) * C::DSS + 8 * h;
        const uint16_t* brow = smem + C::OFF_KT + (32 * dbq + n) * C::KTS + 8 * h;
#pragma unroll
        for (int kc = 0; kc < kBKN / 16; ++kc) {
          if (kc < nkc)
            acc = mfma_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(arow + 16 * kc),
                                     *reinterpret_cast<const bf16x8*>(brow + 16 * kc), acc);
        }
        // acc: lane = feature 32*dbq + n, registers = queries
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow_g = qs0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (qrow_g < N)
            unsafeAtomicAdd(dQh + (size_t)qrow_g * D + 32 * dbq + n, scale * acc[r]);
        }
      }
    }

    if (more) store_qblock<D>(regs, smem, tid);
    __syncthreads();
  }

  // epilogue: dK = scale * dK^T acc, dV = dV^T acc (lane = key, registers = features)
  if (key < N) {
    uint16_t* dkrow = dK + base + (size_t)key * D;
    uint16_t* dvrow = dV + base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        *reinterpret_cast<u32x2*>(dkrow + d0) =
            u32x2{pack_bf16x2(scale * dk[db][4 * g + 0], scale * dk[db][4 * g + 1]),
                  pack_bf16x2(scale * dk[db][4 * g + 2], scale * dk[db][4 * g + 3])};
        *reinterpret_cast<u32x2*>(dvrow + d0) =
            u32x2{pack_bf16x2(dv[db][4 * g + 0], dv[db][4 * g + 1]),
                  pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3])};
      }
  }
}

size_t d_bytes(int BH, int N) { return ((size_t)BH * N * 4 + 255) / 256 * 256; }

template <int D, bool CAUSAL>
hipError_t launch_main(const void* q, const void* k, const void* v, const void* dout,
                       const float* lse, const float* Dv, float* dqacc, void* dk, void* dv,
                       int BH, int N, float scale, hipStream_t stream) {
  using C = BwdCfg<D>;
  const int nkt = (N + kBKN - 1) / kBKN;
  auto kern = bwd_main_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(BH * nkt), dim3(256), C::SMEM_BYTES, stream, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, Dv, dqacc,
                     (uint16_t*)dk, (uint16_t*)dv, BH, N, nkt, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int BH, int N, int d) {
  return d_bytes(BH, N) + (size_t)BH * N * d * 4;
}

// Workspace: D (BH*N floats, rounded up to 256 bytes), then the fp32 dQ
// accumulator (BH*N*d floats).
hipError_t launch_bwd_pre(const void* o, const void* dout, void* ws, int BH, int N, int d,
                          hipStream_t stream) {
  float* Dv = reinterpret_cast<float*>(ws);
  float* dqacc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + d_bytes(BH, N));
  const size_t rows = (size_t)BH * N;
  const size_t threads = rows * (d / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(blocks), dim3(256), 0, stream,
                       (const uint16_t*)o, (const uint16_t*)dout, Dv, dqacc, rows);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(blocks), dim3(256), 0, stream,
                       (const uint16_t*)o, (const uint16_t*)dout, Dv, dqacc, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse, void* dk, void* dv, void* ws, int BH, int N, int d,
                           bool causal, float scale, hipStream_t stream) {
  const float* Dv = reinterpret_cast<const float*>(ws);
  float* dqacc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + d_bytes(BH, N));
  if (d == 128)
    return causal
               ? launch_main<128, true>(q, k, v, dout, lse, Dv, dqacc, dk, dv, BH, N, scale, stream)
               : launch_main<128, false>(q, k, v, dout, lse, Dv, dqacc, dk, dv, BH, N, scale, stream);
  return causal
             ? launch_main<64, true>(q, k, v, dout, lse, Dv, dqacc, dk, dv, BH, N, scale, stream)
             : launch_main<64, false>(q, k, v, dout, lse, Dv, dqacc, dk, dv, BH, N, scale, stream);
}

hipError_t launch_bwd_finalize(void* dq, const void* ws, int BH, int N, int d,
                               hipStream_t stream) {
  const float* dqacc =
      reinterpret_cast<const float*>(reinterpret_cast<const char*>(ws) + d_bytes(BH, N));
  const size_t n8 = (size_t)BH * N * d / 8;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     dqacc, (uint16_t*)dq, n8);
  return hipGetLastError();
}

}  // namespace fa
