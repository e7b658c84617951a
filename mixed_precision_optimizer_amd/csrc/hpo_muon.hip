/*
 * hpo_muon.hip -- gfx950 kernels of the Muon step: momentum and Nesterov
 * gradient, Newton-Schulz orthogonalization on the bf16 matrix cores, and
 * the decayed, scaled master update with the 16-bit write-back.
 *
 * Sources (web pages):
 *   [HANDBOOK]   "优化器：AdamW、Muon 与分布式优化器" (ai-infra-handbooks,
 *                train/algo/optimizer), section on Muon: the momentum, the
 *                Nesterov gradient fed to NS, the NS iteration and its
 *                coefficients, and the update W(1 - lr*wd) - lr*0.2*sqrt(max(A, B))*O
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer),
 *                §1 (EMA momentum), §5.2 (NS, run in bf16), §5.4 (Moonlight
 *                scale and decay), §14.6 (other scales)
 *
 * One batch is a run of same-shape matrices.  Per batch:
 *   momentum   one pass over grad and momentum (chunk table): g = G*inv (*C),
 *              M <- mu M + g (or the EMA form), g~ (Nesterov) to the
 *              workspace, binary64 sum of g~^2 per chunk;     16 B/elem
 *   norm       one workgroup per matrix: fixed-order sum of its chunks
 *   input      X0 = bf16(g~ / (norm + eps)) in the wide orientation (m <= n),
 *              and its transpose, both zero-padded to multiples of 256,
 *              through 64 x 64 LDS tiles;                       8 B/elem
 *   NS step    three bf16 GEMMs on MFMA (v_mfma_f32_32x32x16_bf16, fp32
 *              accumulation), each C = P Q^T with both operands read along
 *              their rows (the matrix cores' natural operand order):
 *                A  = X X^T                  (P = Q = X)
 *                B  = b A + c A A^T          (P = Q = A; A is symmetric)
 *                X' = a X + B X              (P = B, Q = X^T)
 *              the epilogues round A, B and X' to bf16 and write X' both
 *              ways round (X for the next A, X^T for the next B X).
 *   last step  the epilogue keeps O = a X + B X in fp32 and applies
 *              W <- fp32(W * fp32(1 - lr*wd)); W <- fp32(W - fp32(lr*scale) * O)
 *              and the bf16 write-back in place of storing O.
 * Zero padding is a fixed point of the iteration (zero rows and columns of
 * X give zero rows and columns of A, B and X'), so the GEMMs run on whole
 * tiles with no bounds checks.
 *
 * GEMM tiling: a 1024-lane workgroup (4 x 4 wavefronts, one per CU)
 * computes a 256 x 256 tile of C; each wavefront a 64 x 64 block as 2 x 2
 * MFMA tiles of 32 x 32, k in slices of 16.  Operands go straight from
 * global memory into LDS (buffer loads with an LDS destination) in k-stages
 * of 64 (128 B per row), two 64 KB buffers, rows stored with their eight
 * 16-byte pieces permuted by an XOR of the row index so that the MFMA
 * fragment reads (32 rows x 16 B per half-wavefront) hit distinct banks.
 * The k-loop is software-pipelined across the stage barrier: the barrier
 * comes before each stage's last k-slice, whose fragments are already in
 * registers, and the next stage's first fragments are read under that
 * slice's MFMAs.
 * Tiles are handed out XCD by XCD in groups of 8 tile rows.  The epilogues
 * reuse the 128 KB: the bf16 C tile is combined there with its input tile
 * and leaves in whole 128-byte lines, row-major and transposed.
 *
 * Floating point: built with -ffp-contract=off; every elementwise operation
 * rounds on its own, in the order written.
 */
#include <hip/hip_runtime.h>

#include <type_traits>

#include "hpo_muon_impl.h"
#include "hpo_device.h"

namespace hpo {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

/* Pin the interleave of fragment reads and MFMAs with scheduling barriers. */
#ifndef HPO_NS_SCHED
#define HPO_NS_SCHED 1
#endif
/* Raise the wavefront's issue priority while it runs its MFMAs. */
#ifndef HPO_NS_PRIO
#define HPO_NS_PRIO 1
#endif
/* Software-pipeline the k-loop across the stage barrier (see the kernel). */
#ifndef HPO_NS_XBAR
#define HPO_NS_XBAR 1
#endif
/* Tile order: each XCD takes a contiguous run of tiles, rows grouped by this
 * many (0: hardware order). */
#ifndef HPO_NS_GROUP
#define HPO_NS_GROUP 8
#endif
/* NS GEMM tile configurations.  A workgroup of WM x WN wavefronts computes
 * a (WM * TM * 32) x (WN * TN * 32) tile of C, each wavefront TM x TN MFMA
 * tiles of 32 x 32; operands go through LDS in k-stages of BK (STAGES
 * buffers, loads running STAGES - 1 stages ahead); WG is the number of
 * workgroups meant to share a CU (it caps the registers so they fit). */
template <int WM, int WN, int TM, int TN, int BK, int STAGES, int WG>
struct NsTile {
    static constexpr int kWavesM = WM, kWavesN = WN, kTM = TM, kTN = TN, kBK = BK, kStages = STAGES;
    static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
    static constexpr int kBM = WM * TM * 32, kBN = WN * TN * 32;   /* C tile: kBM rows x kBN columns */
    static constexpr int kWavesPerSimd = WG * kWaves / 4;
    static constexpr int kPieces = BK / 8;                /* 16-byte pieces per operand row and stage */
    static constexpr int kRowStride = BK * 2;             /* pieces XOR-swizzled by row (see piece_at) */
    static constexpr int kRowsPerChunk = 1024 / kRowStride;   /* rows one wavefront load (64 x 16 B) fills */
    static constexpr int kStageBytes = (kBM + kBN) * kRowStride;
    static constexpr int kChunks = (kBM + kBN) / kRowsPerChunk;   /* chunks per stage (P rows, then Q rows) */
    static constexpr int kChunksPerWave = kChunks / kWaves;
    /* the epilogue reuses the stages: a bf16 C tile, or half of it in fp32 */
    static constexpr int kEpiBytes = kBM * kBN * 2 > kBM / 2 * kBN * 4 ? kBM * kBN * 2 : kBM / 2 * kBN * 4;
    static constexpr int kLdsBytes = STAGES * kStageBytes > kEpiBytes ? STAGES * kStageBytes : kEpiBytes;
    static_assert(BK == 64 || BK == 32, "direct staging: rows of 128 or 64 B");
    static_assert(kChunks % kWaves == 0, "stage chunks split evenly over the wavefronts");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(kNsPad % kBM == 0 && kNsPad % kBN == 0 && kNsPad % BK == 0, "padding covers the tiles");
    static_assert(kBM == 256 && (kBN == 256 || kBN == 128), "the epilogue's thread maps");
    static_assert(kLdsBytes * WG <= 160 * 1024, "the workgroups of a CU fit its LDS");
};
/* Symmetric outputs (A = XX^T, B = bA + cAA^T) mirror whole tiles: square,
 * 1024 lanes, one workgroup per CU. */
using SymTile = NsTile<4, 4, 2, 2, 64, 2, 1>;
/* General outputs (X' = aX + BX and the last step) take SymTile.
 * HPO_NS_GEN_HALF = 1 selects 256 x 128 tiles of 512 lanes instead, two
 * workgroups per CU (k-stages of HPO_NS_GEN_BK in HPO_NS_GEN_STAGES
 * buffers), so that one workgroup's barriers and stores could overlap the
 * other's MFMAs.  Measured on the MLP batch it is slower (X' = aX + BX at
 * 920-940 TFLOP/s against 1135): the k-stages of 32 double the barriers and
 * the narrower tile reads 1.5x the operand bytes per flop. */
#ifndef HPO_NS_GEN_HALF
#define HPO_NS_GEN_HALF 0
#endif
#ifndef HPO_NS_GEN_BK
#define HPO_NS_GEN_BK 32
#endif
#ifndef HPO_NS_GEN_STAGES
#define HPO_NS_GEN_STAGES 2
#endif
#if HPO_NS_GEN_HALF
using GenTile = NsTile<4, 2, 2, 2, HPO_NS_GEN_BK, HPO_NS_GEN_STAGES, 2>;
#else
using GenTile = SymTile;
#endif
constexpr int kTile = 64;              /* transpose tile of the input kernel */

/* ---------------------------------------------------------------------- */
/* gates and per-step values                                              */
/* ---------------------------------------------------------------------- */
__device__ __forceinline__ bool gate_open(const MuonGate& g)
{
    if (g.dev) {
        /* the finalize has decided and counted the step (t = applied_steps, in the window) */
        if (!g.st->applied)
            return false;
        const int64_t j = g.st->applied_steps - g.t_first;
        return j >= 0 && j < g.window;
    }
    return !(g.d_found != nullptr && *g.d_found != 0);
}

struct GradVals {
    float inv_scale;
    float C;
    bool clip;
};

/* Unscale factor and clip coefficient ([OPT-INFRA] §11.1): the same global
 * norm and rule as the AdamW update of the same step. */
__device__ __forceinline__ GradVals grad_vals(const MuonScalars& sc)
{
    GradVals v;
    float norm = 0.0f;
    if (sc.gate.dev) {
        v.inv_scale = sc.gate.st->step_inv_scale;
        norm = sc.gate.st->grad_norm;
    } else {
        v.inv_scale = sc.inv_scale;
        if (sc.max_norm > 0.0)
            norm = *sc.d_norm;
    }
    v.clip = false;
    v.C = 1.0f;
    if (sc.max_norm > 0.0) {
        const double c = sc.max_norm / (static_cast<double>(norm) + 1e-6);
        if (c < 1.0) {
            v.clip = true;
            v.C = static_cast<float>(c);
        }
    }
    return v;
}

/* ---------------------------------------------------------------------- */
/* momentum + Nesterov gradient                                           */
/* ---------------------------------------------------------------------- */
template <int FORM, bool NEST>
__device__ __forceinline__ float momentum_elem(float G, float& M, const GradVals& k, float mu, float omu, double& acc)
{
    float g = G * k.inv_scale;
    if (k.clip)
        g = g * k.C;
    float gt;
    if constexpr (FORM == HPO_MUON_MOMENTUM_SUM) {
        M = mu * M + g;                 /* [HANDBOOK]: M <- mu M + g */
        gt = NEST ? g + mu * M : M;     /* Nesterov: g + mu M */
    } else {
        M = mu * M + omu * g;           /* [OPT-INFRA] §1: lerp(M, g, 1 - mu) */
        gt = NEST ? omu * g + mu * M : M;
    }
    acc += static_cast<double>(gt) * static_cast<double>(gt);
    return gt;
}

template <int FORM, bool NEST>
__global__ __launch_bounds__(kBlock) void k_muon_momentum(SetView sv, MuonScalars sc, MuonBatch b, float* gt,
                                                         int64_t gt_stride, double* part)
{
    if (!gate_open(sc.gate))
        return;
    const GradVals k = grad_vals(sc);
    const int64_t chunk = b.c0 + blockIdx.x;
    const Chunk c = sv.chunks[chunk];
    const TensorDesc d = sv.tensors[c.tensor];
    const int64_t slot = c.tensor - b.first;
    const float* __restrict__ G = d.grad + c.start;
    float* __restrict__ M = static_cast<float*>(d.exp_avg) + c.start;
    float* __restrict__ O = gt + slot * gt_stride + c.start;
    const int tid = threadIdx.x;
    double acc = 0.0;
    const int64_t nv = c.len / kVec;  /* Muon tensors are 16-byte aligned */
    for (int64_t i = tid; i < nv; i += kBlock) {
        const float4 g4 = reinterpret_cast<const float4*>(G)[i];
        float4 m4 = reinterpret_cast<float4*>(M)[i];
        float4 o4;
        o4.x = momentum_elem<FORM, NEST>(g4.x, m4.x, k, sc.mu, sc.omu, acc);
        o4.y = momentum_elem<FORM, NEST>(g4.y, m4.y, k, sc.mu, sc.omu, acc);
        o4.z = momentum_elem<FORM, NEST>(g4.z, m4.z, k, sc.mu, sc.omu, acc);
        o4.w = momentum_elem<FORM, NEST>(g4.w, m4.w, k, sc.mu, sc.omu, acc);
        reinterpret_cast<float4*>(M)[i] = m4;
        reinterpret_cast<float4*>(O)[i] = o4;
    }
    for (int64_t e = nv * kVec + tid; e < c.len; e += kBlock) {
        float m = M[e];
        O[e] = momentum_elem<FORM, NEST>(G[e], m, k, sc.mu, sc.omu, acc);
        M[e] = m;
    }
    const double tot = block_sum<kBlock>(acc);
    if (tid == 0)
        part[chunk] = tot;
}

/* Per-matrix fold of the chunk sums: dnorm = fp32(fp32(sqrt(sum)) + eps). */
__global__ __launch_bounds__(kBlock) void k_muon_norm(const MuonInfo* info, MuonGate gate, int32_t first,
                                                     const double* part, float eps, float* dnorm)
{
    if (!gate_open(gate))
        return;
    const int32_t mat = first + static_cast<int32_t>(blockIdx.x);
    const MuonInfo in = info[mat];
    double acc = 0.0;
    for (int32_t i = threadIdx.x; i < in.n_chunks; i += kBlock)
        acc += part[in.first_chunk + i];
    const double tot = block_sum<kBlock>(acc);
    if (threadIdx.x == 0)
        dnorm[mat] = static_cast<float>(sqrt(tot)) + eps;
}

/* Sum of squares of a plain fp32 matrix (the standalone NS entry). */
__global__ __launch_bounds__(kBlock) void k_sumsq_rows(const float* G, int64_t n, int64_t per_block, double* part)
{
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per_block;
    const int64_t hi = lo + per_block < n ? lo + per_block : n;
    double acc = 0.0;
    for (int64_t e = lo + threadIdx.x; e < hi; e += kBlock) {
        const double x = G[e];
        acc += x * x;
    }
    const double tot = block_sum<kBlock>(acc);
    if (threadIdx.x == 0)
        part[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kBlock) void k_sumsq_fold(const double* part, int32_t n, float eps, float* dnorm)
{
    double acc = 0.0;
    for (int32_t i = threadIdx.x; i < n; i += kBlock)
        acc += part[i];
    const double tot = block_sum<kBlock>(acc);
    if (threadIdx.x == 0)
        dnorm[0] = static_cast<float>(sqrt(tot)) + eps;
}

/* ---------------------------------------------------------------------- */
/* NS input: X0 = bf16(g~ / d) both ways round                            */
/* ---------------------------------------------------------------------- */
/* grid (Cp / 64, Rp / 64, count) over the padded natural shape.  Natural
 * row-major g~ (R x C) is read along its rows; the bf16 tile goes out once
 * in the natural orientation ("copy") and once transposed.  In the wide
 * orientation the copy is X (not transposed) or X^T (transposed matrix). */
__global__ __launch_bounds__(kBlock) void k_muon_ns_input(const float* src, int64_t src_stride, const float* dnorm,
                                                         int32_t dnorm_first, int64_t R, int64_t C,
                                                         uint16_t* copy, int64_t ld_copy, int64_t s_copy,
                                                         uint16_t* trans, int64_t ld_trans, int64_t s_trans,
                                                         MuonGate gate)
{
    if (!gate_open(gate))
        return;
    __shared__ __attribute__((aligned(4))) uint16_t tile[kTile][kTile + 2];
    const int64_t z = blockIdx.z;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTile;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const float d = dnorm[dnorm_first + z];
    const float* __restrict__ S = src + z * src_stride;
    const int tid = threadIdx.x;
    /* a thread takes column pairs (one 4-byte LDS write each); all of its
     * loads are issued before the first use */
    constexpr int kPairs = kTile * kTile / 2 / kBlock;
    float x0[kPairs], x1[kPairs];
    /* even rows on an 8-byte aligned base: each pair is one 8-byte load
     * (gc is even, so gc < C means gc + 1 < C) */
    const bool pairs = (C & 1) == 0 && (reinterpret_cast<uintptr_t>(S) & 7) == 0;
    if (pairs) {
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            const int e = tid + k * kBlock;
            const int r = e / (kTile / 2), c = (e % (kTile / 2)) * 2;
            const int64_t gr = r0 + r, gc = c0 + c;
            float2 v = make_float2(0.0f, 0.0f);
            if (gr < R && gc < C)
                v = *reinterpret_cast<const float2*>(S + gr * C + gc);
            x0[k] = v.x;
            x1[k] = v.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            const int e = tid + k * kBlock;
            const int r = e / (kTile / 2), c = (e % (kTile / 2)) * 2;
            const int64_t gr = r0 + r, gc = c0 + c;
            x0[k] = gr < R && gc < C ? S[gr * C + gc] : 0.0f;
            x1[k] = gr < R && gc + 1 < C ? S[gr * C + gc + 1] : 0.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
        const int e = tid + k * kBlock;
        const int r = e / (kTile / 2), c = (e % (kTile / 2)) * 2;
        const uint32_t lo = bf16_rne_bits(x0[k] / d), hi = bf16_rne_bits(x1[k] / d);
        *reinterpret_cast<uint32_t*>(&tile[r][c]) = lo | (hi << 16);
    }
    __syncthreads();
    uint16_t* __restrict__ Cp = copy + z * s_copy;
    uint16_t* __restrict__ Tp = trans + z * s_trans;
    /* 64 rows x 8 pieces of 8 bf16 (16 B) each way */
#pragma unroll
    for (int q = 0; q < kTile * kTile / 8 / kBlock; ++q) {
        const int e = tid + q * kBlock;
        const int r = e / 8, p = (e % 8) * 8;
        u32x4_t v;
        v.x = tile[r][p + 0] | (static_cast<uint32_t>(tile[r][p + 1]) << 16);
        v.y = tile[r][p + 2] | (static_cast<uint32_t>(tile[r][p + 3]) << 16);
        v.z = tile[r][p + 4] | (static_cast<uint32_t>(tile[r][p + 5]) << 16);
        v.w = tile[r][p + 6] | (static_cast<uint32_t>(tile[r][p + 7]) << 16);
        *reinterpret_cast<u32x4_t*>(Cp + (r0 + r) * ld_copy + c0 + p) = v;
        u32x4_t t;
        t.x = tile[p + 0][r] | (static_cast<uint32_t>(tile[p + 1][r]) << 16);
        t.y = tile[p + 2][r] | (static_cast<uint32_t>(tile[p + 3][r]) << 16);
        t.z = tile[p + 4][r] | (static_cast<uint32_t>(tile[p + 5][r]) << 16);
        t.w = tile[p + 6][r] | (static_cast<uint32_t>(tile[p + 7][r]) << 16);
        *reinterpret_cast<u32x4_t*>(Tp + (c0 + r) * ld_trans + r0 + p) = t;
    }
}

/* ---------------------------------------------------------------------- */
/* NS GEMM: C = P Q^T on bf16 MFMA with fused epilogues                   */
/* ---------------------------------------------------------------------- */
enum Epi : int {
    kEpiGram = 0,    /* C = bf16(acc)                              A = X X^T      */
    kEpiPoly = 1,    /* C = bf16(b * P[i][j] + c * acc)           B = b A + c A A */
    kEpiStep = 2,    /* X = bf16(a * X + acc) in place, and X^T    X' = a X + B X */
    kEpiUpdate = 3,  /* O = a * X + acc (fp32) -> master / param update */
    kEpiOut = 4,     /* O = a * X + acc (fp32) -> out, natural layout */
};

struct GemmArgs {
    const uint16_t* P;
    const uint16_t* Q;
    int64_t ldp, sp, ldq, sq;
    int32_t K;
    int32_t nt;          /* symmetric outputs: tiles per side */
    int32_t nx, ny;      /* general outputs: tiles per row, per column */
    int32_t first;       /* matrix index of slot 0 (update epilogue) */
    uint16_t* C;         /* gram / poly output */
    int64_t ldc, sc;
    uint16_t* X;         /* step / update / out: X (wide, bf16) */
    int64_t ldx, sx;
    uint16_t* XT;        /* step: next X^T */
    int64_t ldxt, sxt;
    const uint16_t* XS;  /* step / update / out: X^T (rows are columns of X), read by the epilogue */
    int64_t ldxs, sxs;
    float a, b, c;
    int64_t R, Cn;       /* update / out: natural shape; the C tile is in natural orientation */
    float* out;          /* out epilogue */
    const TensorDesc* desc;
    const MuonInfo* info;
    MuonGate gate;
};

__device__ __forceinline__ float bf16v(uint16_t b) { return bf16_to_f32(b); }

/* Scale of the orthogonalized update, binary64 ([OPT-INFRA] §5.4 Moonlight:
 * 0.2 * sqrt(max(A, B)); §14.6: the spectral, shape and unit-RMS bases times
 * an extra factor, with fan_out = rows and fan_in = cols). */
__device__ __forceinline__ double update_scale(int64_t rows, int64_t cols, const MuonUpdate& up)
{
    const double r = static_cast<double>(rows), c = static_cast<double>(cols);
    double base;
    if (up.scale_mode == HPO_MUON_SCALE_SHAPE)
        base = sqrt(r / c > 1.0 ? r / c : 1.0);
    else if (up.scale_mode == HPO_MUON_SCALE_UNIT_RMS)
        base = sqrt(r / c);
    else
        base = sqrt(r > c ? r : c);
    return base * up.extra_scale;
}

/* Byte offset of 16-byte piece p of LDS row r.  Direct staging stores row r's
 * pieces permuted by an XOR with (r & 7) ^ ((r >> 3) & 1): the 16 (or 8) rows
 * that one fragment read serves per LDS cycle then land on distinct banks
 * whether the LDS has 64 or 32 four-byte banks. */
template <int BK>
__device__ __forceinline__ int swizzle(int r)
{
    if constexpr (BK == 64)
        return (r & 7) ^ ((r >> 3) & 1);   /* 8 pieces per row */
    else
        return (r ^ (r >> 2)) & 3;         /* 4 pieces per row */
}

template <int BK>
__device__ __forceinline__ int piece_at(int r, int p)
{
    return r * (BK * 2) + ((p ^ swizzle<BK>(r)) << 4);
}

/* One wavefront load of 64 x 16 bytes from a buffer straight into LDS: lane
 * l's piece lands at dst + 16 l.  (A plain device function: the host pass
 * of a kernel template does not take this builtin in a dependent context.) */
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

/* Tile of the t-th workgroup in dispatch order.  Workgroups go to the 8
 * XCDs round-robin; the remap gives XCD x one contiguous run of tile numbers
 * (so the tiles running on one XCD share operand panels in its L2).  Tile
 * numbers then walk groups of HPO_NS_GROUP tile rows column by column
 * (general outputs), or the upper triangle row by row (symmetric outputs,
 * tiles with ty <= tx only). */
__device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t n)
{
#if HPO_NS_GROUP
    constexpr int64_t kXcd = 8;
    const int64_t x = b % kXcd, k = b / kXcd;
    const int64_t q = n / kXcd, r = n % kXcd;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
#else
    (void)n;
    return b;
#endif
}

template <bool SYM>
__device__ __forceinline__ void tile_of(const GemmArgs& g, int64_t& ty, int64_t& tx)
{
    if constexpr (SYM) {
        const int32_t nt = g.nt;
        int64_t t = xcd_contiguous(blockIdx.x, static_cast<int64_t>(nt) * (nt + 1) / 2);
        int64_t y = 0, row = nt;
        while (t >= row) {
            t -= row;
            ++y;
            --row;
        }
        ty = y;
        tx = y + t;
    } else {
        const int64_t nx = g.nx, ny = g.ny;
        const int64_t t = xcd_contiguous(blockIdx.x, nx * ny);
#if HPO_NS_GROUP
        const int64_t G = HPO_NS_GROUP;
        const int64_t group = t / (G * nx);
        const int64_t first = group * G;
        const int64_t rows = ny - first < G ? ny - first : G;
        const int64_t within = t - group * G * nx;
        ty = first + within % rows;
        tx = within / rows;
#else
        ty = t / nx;
        tx = t % nx;
#endif
    }
}

template <int EPI, bool SYM, class T>
__global__ __launch_bounds__(T::kThreads, T::kWavesPerSimd) void k_ns_gemm(GemmArgs g, MuonUpdate up)
{
    constexpr int kWavesN = T::kWavesN, kTM = T::kTM, kTN = T::kTN, kBK = T::kBK, kStages = T::kStages;
    constexpr int kBM = T::kBM, kBN = T::kBN, kNsThreads = T::kThreads;
    constexpr int kRowStride = T::kRowStride, kPieces = T::kPieces, kRowsPerChunk = T::kRowsPerChunk;
    constexpr int kChunksPerWave = T::kChunksPerWave;
    static_assert(!SYM || kBM == kBN, "symmetric outputs mirror square tiles");
    if (!gate_open(g.gate))
        return;
    __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
    const int64_t z = blockIdx.z;
    int64_t ty, tx;
    tile_of<SYM>(g, ty, tx);
    const int64_t row0 = ty * kBM;
    const int64_t col0 = tx * kBN;
    const uint16_t* __restrict__ P = g.P + z * g.sp + row0 * g.ldp;
    const uint16_t* __restrict__ Q = g.Q + z * g.sq + col0 * g.ldq;
    const int tid = threadIdx.x;
    /* the wavefront index is uniform: keep it scalar so chunk choices, descriptors and the LDS
     * destination of each load stay in SGPRs */
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    /* Operands go straight from global memory into LDS.  One wavefront load
     * fills 1 KB = kRowsPerChunk rows of one stage, lane l landing in row
     * l / kPieces, physical piece l % kPieces; the lane fetches the logical
     * piece that the swizzle puts there.  gfx9 buffer descriptor, last dword:
     * 32-bit data format, raw (untyped, unswizzled) addressing.  Each operand
     * panel is the tile's rows (P) or columns (Q) from its first one, so every
     * offset fits 32 bits. */
    constexpr int kRawBuffer = 0x00020000;
    static_assert(int64_t{kBM > kBN ? kBM : kBN} * ns_pad(HPO_MUON_MAX_DIM) * 2 <= INT32_MAX,
                  "an operand panel of the widest matrix fits 32-bit buffer offsets");
    const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(P), 0, static_cast<int>(kBM * g.ldp * 2), kRawBuffer);
    const __amdgpu_buffer_rsrc_t rsQ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Q), 0, static_cast<int>(kBN * g.ldq * 2), kRawBuffer);
    /* LDS: the P panels of all stages, then the Q panels ([P0 P1 .. Q0 Q1 ..]),
     * so a fragment address of one stage and the same address of the next
     * differ by kBM * kRowStride (32 KB), within a DS instruction's offset */
    constexpr int kChunksP = kBM / kRowsPerChunk;   /* chunks holding P rows */
    auto p_stage = [&](int s) { return lds + s * (kBM * kRowStride); };
    auto q_stage = [&](int s) { return lds + kStages * (kBM * kRowStride) + s * (kBN * kRowStride); };
    int voff[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        const int c = wave * kChunksPerWave + i;
        const int r = c * kRowsPerChunk + lane / kPieces;
        const int p = (lane % kPieces) ^ swizzle<kBK>(r);
        voff[i] = r < kBM ? (r * static_cast<int>(g.ldp) + p * 8) * 2 : ((r - kBM) * static_cast<int>(g.ldq) + p * 8) * 2;
    }
    auto gload = [&](int s, int64_t k0) {
#pragma unroll
        for (int i = 0; i < kChunksPerWave; ++i) {
            const int c = wave * kChunksPerWave + i;
            const bool is_p = c * kRowsPerChunk < kBM;   /* uniform per chunk */
            char* dst = is_p ? p_stage(s) + c * 1024 : q_stage(s) + (c - kChunksP) * 1024;
            buffer_load_lds16(is_p ? rsP : rsQ, dst, voff[i], static_cast<int>(k0 * 2));
        }
    };
    const int wm = (wave / kWavesN) * 32 * kTM, wn = (wave % kWavesN) * 32 * kTN;
    const int frow = lane & 31, fhalf = lane >> 5;
    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            acc[i][j] = f32x16_t{};
    /* One k-stage from LDS buffer s: fragments of slice kk + 1 are read
     * while the MFMAs of slice kk run; the scheduling barriers keep the
     * compiler from sinking the reads next to their uses. */
    auto compute = [&](int s) {
        const char* Ps = p_stage(s);
        const char* Qs = q_stage(s);
        bf16x8_t fa[2][kTM], fb[2][kTN];
        auto fload = [&](int kk, int buf) {
            const int piece = kk * 2 + fhalf;  /* lanes 0-31: k 0..7 of the slice, 32-63: k 8..15 */
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                fa[buf][i] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Ps + piece_at<kBK>(wm + 32 * i + frow, piece)));
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                fb[buf][j] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Qs + piece_at<kBK>(wn + 32 * j + frow, piece)));
        };
        fload(0, 0);
#if HPO_NS_PRIO
        __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < kBK / 16)
                fload(kk + 1, cur ^ 1);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
#if HPO_NS_SCHED
            if (kk + 1 < kBK / 16) {
                /* the next slice's kTM + kTN reads spread over this slice's kTM * kTN MFMAs */
                constexpr int kReads = kTM + kTN, kPer = kTM * kTN / kReads, kRest = kTM * kTN - kPer * kReads;
#pragma unroll
                for (int q = 0; q < kReads; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      /* one DS read */
                    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);   /* MFMAs */
                }
                if (kRest > 0)
                    __builtin_amdgcn_sched_group_barrier(0x008, kRest, 0);
            }
#endif
        }
#if HPO_NS_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
    };
    const int nk = g.K / kBK;
    /* the cross-barrier pipeline needs two stages of four k-slices */
    constexpr bool kXbar = HPO_NS_XBAR && kBK == 64 && kStages == 2;
    if constexpr (kXbar) {
        /* Two stages, the barrier moved inside the stream of k-slices.  The
         * fragments of slice kk + 1 are read while the MFMAs of slice kk run, across
         * stage boundaries too: before the last slice of stage kt (its fragments
         * already in registers) a wavefront waits for its own LDS reads of that
         * buffer and its own loads of stage kt + 1, then the barrier makes both
         * true for every wavefront.  Stage kt + 2 then goes into the retired
         * buffer and the first fragments of stage kt + 1 are read while the last
         * MFMAs of stage kt run, so the matrix pipe is busy across the barrier. */
        constexpr int kSlices = kBK / 16;
        bf16x8_t fa[2][kTM], fb[2][kTN];
        auto fload = [&](int s, int kk, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            const char* Ps = p_stage(s);
            const char* Qs = q_stage(s);
            const int piece = kk * 2 + fhalf;  /* lanes 0-31: k 0..7 of the slice, 32-63: k 8..15 */
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                fa[buf][i] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Ps + piece_at<kBK>(wm + 32 * i + frow, piece)));
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                fb[buf][j] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Qs + piece_at<kBK>(wn + 32 * j + frow, piece)));
        };
        auto mfmas = [&](auto bufc) {
            constexpr int buf = decltype(bufc)::value;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
        };
        auto interleave = [&]() {
            __builtin_amdgcn_sched_barrier(0);   /* one scheduling region per slice */
#if HPO_NS_SCHED
            /* the kTM + kTN reads of the next slice spread over this slice's kTM * kTN MFMAs */
            constexpr int kReads = kTM + kTN, kPer = kTM * kTN / kReads, kRest = kTM * kTN - kPer * kReads;
#pragma unroll
            for (int q = 0; q < kReads; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      /* one DS read */
                __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);   /* MFMAs */
            }
            if (kRest > 0)
                __builtin_amdgcn_sched_group_barrier(0x008, kRest, 0);
#endif
            __builtin_amdgcn_sched_barrier(0);
        };
        /* gfx9 s_waitcnt encoding: vmcnt [3:0] and [15:14], expcnt [6:4],
         * lgkmcnt [11:8].  The barriers are the bare instruction:
         * __syncthreads()'s release fence would also wait for every outstanding
         * load (vmcnt(0)) and drain the pipeline. */
        constexpr int kOne = kChunksPerWave;   /* one stage of this wavefront's loads */
        static_assert(kOne < 64, "vmcnt range");
        constexpr int kWaitOne = 0x0070 | (kOne & 15) | ((kOne >> 4) << 14);
        gload(0, 0);
        if (nk > 1)
            gload(1, kBK);
        if (nk > 1)
            __builtin_amdgcn_s_waitcnt(kWaitOne);   /* stage 0 has landed (stage 1 may still be in flight) */
        else
            __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        using F0 = std::integral_constant<int, 0>;
        using F1 = std::integral_constant<int, 1>;
        fload(0, 0, F0{});
        /* nk is even and at least 4 (K is a multiple of 256): two stages per
         * trip, so that each stage's buffer index is a constant, and the last two
         * stages peeled, so that no branch inside the loop splits the
         * accumulators' live range.  kMode: 0 a stage that loads stage kt + 2,
         * 1 the last but one (no later stage to load), 2 the last (no barrier). */
        auto stage = [&](int kt, auto sbuf, auto mode) {
            constexpr int s = decltype(sbuf)::value;
            constexpr int kMode = decltype(mode)::value;
#if HPO_NS_PRIO
            __builtin_amdgcn_s_setprio(1);
#endif
            static_assert(kSlices == 4, "four k-slices per stage");
            fload(s, 1, F1{});
            mfmas(F0{});
            interleave();
            fload(s, 2, F0{});
            mfmas(F1{});
            interleave();
            fload(s, 3, F1{});
            mfmas(F0{});
            interleave();
            if constexpr (kMode < 2) {
#if HPO_NS_PRIO
                __builtin_amdgcn_s_setprio(0);
#endif
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0x0070);   /* own reads of buffer s, own loads of stage kt + 1 */
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kMode == 0)
                    gload(s, static_cast<int64_t>(kt + 2) * kBK);
                __builtin_amdgcn_sched_barrier(0);
#if HPO_NS_PRIO
                __builtin_amdgcn_s_setprio(1);
#endif
                fload(s ^ 1, 0, F0{});   /* the next stage's first slice, under this stage's last MFMAs */
                mfmas(F1{});
                interleave();
            } else {
                mfmas(F1{});
            }
#if HPO_NS_PRIO
            __builtin_amdgcn_s_setprio(0);
#endif
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        int kt = 0;
        for (; kt + 2 < nk; kt += 2) {
            stage(kt, S0{}, std::integral_constant<int, 0>{});
            stage(kt + 1, S1{}, std::integral_constant<int, 0>{});
        }
        stage(kt, S0{}, std::integral_constant<int, 1>{});
        stage(kt + 1, S1{}, std::integral_constant<int, 2>{});
    } else {
        /* Stages kt .. kt + kStages - 2 are in flight while stage kt is
         * computed.  At the top of iteration kt a wavefront waits until its own
         * loads of stage kt have landed (vmcnt counts its outstanding loads, in
         * issue order, kChunksPerWave per stage), the barrier makes that true
         * for every wavefront and retires buffer (kt - 1) % kStages, which then
         * receives stage kt + kStages - 1. */
        for (int st = 0; st < kStages - 1 && st < nk; ++st)
            gload(st, static_cast<int64_t>(st) * kBK);
        for (int kt = 0; kt < nk; ++kt) {
            /* gfx9 s_waitcnt encoding: vmcnt [3:0] and [15:14], expcnt [6:4],
             * lgkmcnt [11:8].  lgkmcnt(0): this wavefront's LDS reads of the
             * buffer about to be refilled have completed.  The barrier is the
             * bare instruction: __syncthreads()'s release fence would also wait
             * for every outstanding load (vmcnt(0)) and drain the pipeline. */
            constexpr int kAhead = (kStages - 2) * kChunksPerWave;
            constexpr int kWaitAhead = 0x0070 | (kAhead & 15) | ((kAhead >> 4) << 14);
            static_assert(kAhead < 64, "vmcnt range");
            __builtin_amdgcn_sched_barrier(0);
            if (kt + kStages - 2 < nk)
                __builtin_amdgcn_s_waitcnt(kWaitAhead);
            else
                __builtin_amdgcn_s_waitcnt(0x0070);   /* the tail: nothing later was issued */
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            const int nxt = kt + kStages - 1;
            if (nxt < nk)
                gload(nxt % kStages, static_cast<int64_t>(nxt) * kBK);
#if HPO_NS_SCHED
            __builtin_amdgcn_sched_barrier(0);
#endif
            compute(kt % kStages);
        }
    }

    /* Staged epilogue.  acc[ti][tj][r] holds C[i][j] (tile coordinates) with
     * i = wm + 32 ti + 8 (r / 4) + 4 (lane / 32) + r % 4 and
     * j = wn + 32 tj + lane % 32: four consecutive rows of one column per
     * group of four registers.  The stage buffers are free once every
     * wavefront has left the k-loop; they then hold the bf16 tile
     * column-major (Tt[j][i] = C[i][j]), so such a group is one 8-byte LDS
     * access, the transposed copy of the tile leaves with 16-byte LDS reads
     * and the row-major copy gathers 8 x 4 blocks with 8-byte reads.  The
     * 16-byte chunks of column j are XOR-permuted by f(j) = (j ^ j / 8) % 16:
     * each of the three access patterns then spreads over all banks.  For the
     * master update the fp32 output goes through LDS half a tile at a time
     * (row-major, a 32-float XOR that separates the two row halves of a
     * wavefront's access).  Global traffic is whole 16-byte pieces, eight
     * lanes per 128-byte line. */
    {
        constexpr int kCPR = kBM / 8;                        /* 16-byte chunks per tile column */
        constexpr int kEpiPieces = kBN * kCPR / kNsThreads;  /* 16-byte pieces per thread */
        constexpr int kJB = kBN / 8;                         /* 8-column blocks per tile row */
        constexpr int kBlocks = (kBM / 4) * kJB / kNsThreads;   /* 4 x 8 blocks per thread */
        static_assert(kEpiPieces * kNsThreads == kBN * kCPR && kBlocks * kNsThreads == (kBM / 4) * kJB, "whole pieces");
        static_assert(kCPR >= 16 && (kJB == 16 || kJB == 32), "bank maps");
        uint16_t* Tt = reinterpret_cast<uint16_t*>(lds);
        float* T32 = reinterpret_cast<float*>(lds);
        /* element offset of C[i][j] */
        auto tt = [](int j, int i) {
            return j * kBM + ((((i >> 3) ^ ((j ^ (j >> 3)) & 15)) & (kCPR - 1)) << 3) + (i & 7);
        };
        /* Tt[j][.] = src[j][.] : src holds C^T row-major (row j = column j of C) */
        auto stage_in = [&](const uint16_t* src, int64_t ld) {
            u32x4_t v[kEpiPieces];   /* all loads in flight before the first LDS write */
#pragma clang loop unroll(full)
            for (int k = 0; k < kEpiPieces; ++k) {
                const int idx = tid + k * kNsThreads, j = idx / kCPR, i = (idx % kCPR) * 8;
                v[k] = *reinterpret_cast<const u32x4_t*>(src + j * ld + i);
            }
#pragma clang loop unroll(full)
            for (int k = 0; k < kEpiPieces; ++k) {
                const int idx = tid + k * kNsThreads, j = idx / kCPR, i = (idx % kCPR) * 8;
                *reinterpret_cast<u32x4_t*>(Tt + tt(j, i)) = v[k];
            }
        };
        /* dst[j][i] = C[i][j] */
        auto store_t = [&](uint16_t* dst, int64_t ld) {
#pragma clang loop unroll(full)
            for (int k = 0; k < kEpiPieces; ++k) {
                const int idx = tid + k * kNsThreads, j = idx / kCPR, i = (idx % kCPR) * 8;
                *reinterpret_cast<u32x4_t*>(dst + j * ld + i) = *reinterpret_cast<const u32x4_t*>(Tt + tt(j, i));
            }
        };
        /* dst[i][j] = C[i][j]: a thread moves 4 rows x 8 columns per block;
         * of 32 consecutive blocks, the lowest bit picks the row quad (par)
         * and the next four 16 of the column blocks (jb) */
        auto store_n = [&](uint16_t* dst, int64_t ld) {
#pragma clang loop unroll(full)
            for (int k = 0; k < kBlocks; ++k) {
                const int bidx = tid + k * kNsThreads;
                const int rest = bidx >> 5;
                const int par = bidx & 1, jb = ((bidx >> 1) & 15) | ((rest % (kJB / 16)) << 4), ic = rest / (kJB / 16);
                const int i0 = 8 * ic + 4 * par, j0 = 8 * jb;
                u32x2_t v[8];
#pragma clang loop unroll(full)
                for (int e = 0; e < 8; ++e)
                    v[e] = *reinterpret_cast<const u32x2_t*>(Tt + tt(j0 + e, i0));
#pragma clang loop unroll(full)
                for (int r = 0; r < 4; ++r) {
                    const int sh = 16 * (r & 1);
                    auto el = [&](int e) { return ((r < 2 ? v[e].x : v[e].y) >> sh) & 0xffffu; };
                    u32x4_t o;
                    o.x = el(0) | (el(1) << 16);
                    o.y = el(2) | (el(3) << 16);
                    o.z = el(4) | (el(5) << 16);
                    o.w = el(6) | (el(7) << 16);
                    *reinterpret_cast<u32x4_t*>(dst + (i0 + r) * ld + j0) = o;
                }
            }
        };
        const int lcol = lane & 31, lrow4 = 4 * (lane >> 5);
        auto pack4 = [](float a0, float a1, float a2, float a3) {
            u32x2_t t;
            t.x = bf16_rne_bits(a0) | (bf16_rne_bits(a1) << 16);
            t.y = bf16_rne_bits(a2) | (bf16_rne_bits(a3) << 16);
            return t;
        };
        auto unpack = [](u32x2_t t, int e) {
            const uint32_t w = e < 2 ? t.x : t.y;
            return bf16v(static_cast<uint16_t>(e & 1 ? w >> 16 : w & 0xffffu));
        };
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();   /* every wavefront is past its last fragment read */
        if constexpr (EPI == kEpiGram || EPI == kEpiPoly) {
            const bool diag = SYM && ty == tx;
            if constexpr (EPI == kEpiPoly) {
                /* A is symmetric and stored whole: column j of the tile is row col0 + j */
                stage_in(g.P + z * g.sp + col0 * g.ldp + row0, g.ldp);
                __syncthreads();
            }
#pragma clang loop unroll(full)
            for (int ti = 0; ti < kTM; ++ti)
#pragma clang loop unroll(full)
                for (int tj = 0; tj < kTN; ++tj) {
#pragma clang loop unroll(full)
                    for (int q = 0; q < 4; ++q) {
                        const int i = wm + 32 * ti + 8 * q + lrow4, j = wn + 32 * tj + lcol;
                        u32x2_t* pt = reinterpret_cast<u32x2_t*>(Tt + tt(j, i));
                        float x[4];
#pragma clang loop unroll(full)
                        for (int e = 0; e < 4; ++e)
                            x[e] = acc[ti][tj][4 * q + e];
                        if constexpr (EPI == kEpiPoly) {
                            const u32x2_t av = *pt;
#pragma clang loop unroll(full)
                            for (int e = 0; e < 4; ++e) {
                                const float bv = g.b * unpack(av, e);
                                const float cv = g.c * x[e];
                                x[e] = bv + cv;
                            }
                        }
                        *pt = pack4(x[0], x[1], x[2], x[3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);   /* one 32 x 32 block at a time */
                }
            __syncthreads();
            if (diag) {
                /* the lower triangle of a diagonal tile is the mirror of its upper one */
#pragma clang loop unroll(full)
                for (int k = 0; k < kBM * kBN / kNsThreads; ++k) {
                    const int idx = tid + k * kNsThreads, j = idx / kBM, i = idx % kBM;
                    if (i > j)
                        Tt[tt(j, i)] = Tt[tt(i, j)];
                }
                __syncthreads();
            }
            uint16_t* Cz = g.C + z * g.sc;
            store_n(Cz + row0 * g.ldc + col0, g.ldc);
            if (SYM && !diag)
                store_t(Cz + col0 * g.ldc + row0, g.ldc);   /* the mirror tile */
        } else if constexpr (EPI == kEpiStep) {
            stage_in(g.XS + z * g.sxs + col0 * g.ldxs + row0, g.ldxs);
            __syncthreads();
#pragma clang loop unroll(full)
            for (int ti = 0; ti < kTM; ++ti)
#pragma clang loop unroll(full)
                for (int tj = 0; tj < kTN; ++tj) {
#pragma clang loop unroll(full)
                    for (int q = 0; q < 4; ++q) {
                        const int i = wm + 32 * ti + 8 * q + lrow4, j = wn + 32 * tj + lcol;
                        u32x2_t* pt = reinterpret_cast<u32x2_t*>(Tt + tt(j, i));
                        const u32x2_t xv = *pt;
                        float x[4];
#pragma clang loop unroll(full)
                        for (int e = 0; e < 4; ++e) {
                            const float ax = g.a * unpack(xv, e);
                            x[e] = ax + acc[ti][tj][4 * q + e];
                        }
                        *pt = pack4(x[0], x[1], x[2], x[3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            __syncthreads();
            store_n(g.X + z * g.sx + row0 * g.ldx + col0, g.ldx);
            store_t(g.XT + z * g.sxt + col0 * g.ldxt + row0, g.ldxt);
        } else {
            /* last step: O = a X + acc in fp32 (registers), then the master
             * update (or O itself) streamed by rows, half a tile at a time.
             * The per-matrix factors are wave-uniform: kept in scalar
             * registers, computed before the tile work. */
            float k1 = 0.0f, k2 = 0.0f;
            float* __restrict__ W = nullptr;
            uint16_t* __restrict__ Pm = nullptr;
            if constexpr (EPI == kEpiUpdate) {
                const int32_t mat = g.first + static_cast<int32_t>(z);
                const MuonInfo in = g.info[mat];
                const double lr = up.lr[in.group], wd = up.wd[in.group];
                k1 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                         __builtin_bit_cast(int, static_cast<float>(1.0 - lr * wd))));
                k2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                         __builtin_bit_cast(int, static_cast<float>(lr * update_scale(in.rows, in.cols, up)))));
                W = g.desc[mat].master;
                Pm = up.param_dtype == HPO_PARAM_FP32 ? nullptr : static_cast<uint16_t*>(g.desc[mat].param);
            }
            __builtin_amdgcn_sched_barrier(0);
            stage_in(g.XS + z * g.sxs + col0 * g.ldxs + row0, g.ldxs);
            __syncthreads();
#pragma clang loop unroll(full)
            for (int ti = 0; ti < kTM; ++ti)
#pragma clang loop unroll(full)
                for (int tj = 0; tj < kTN; ++tj) {
#pragma clang loop unroll(full)
                    for (int q = 0; q < 4; ++q) {
                        const int i = wm + 32 * ti + 8 * q + lrow4, j = wn + 32 * tj + lcol;
                        const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(Tt + tt(j, i));
#pragma clang loop unroll(full)
                        for (int e = 0; e < 4; ++e) {
                            const float ax = g.a * unpack(xv, e);
                            acc[ti][tj][4 * q + e] = ax + acc[ti][tj][4 * q + e];
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            /* whole float4 pieces when every row starts 16-byte aligned (W always is) */
            const bool vec = (g.Cn & 3) == 0 &&
                             (EPI == kEpiUpdate || (reinterpret_cast<uintptr_t>(g.out) & 15) == 0);
            constexpr int kHalf = kBM / 2;
            /* row-major half tile; column bit 5 flipped on rows with bit 2 set */
            auto t32 = [](int i, int j) { return i * kBN + (j ^ (((i >> 2) & 1) << 5)); };
            static_assert(kHalf % (32 * kTM) == 0, "a wavefront's rows lie in one half");
#pragma clang loop unroll(full)
            for (int h = 0; h < 2; ++h) {
                __syncthreads();   /* Tt / the previous half is no longer read */
                if (wm / kHalf == h) {
#pragma clang loop unroll(full)
                    for (int ti = 0; ti < kTM; ++ti)
#pragma clang loop unroll(full)
                        for (int tj = 0; tj < kTN; ++tj)
#pragma clang loop unroll(full)
                            for (int r = 0; r < 16; ++r) {
                                const int i = wm - h * kHalf + 32 * ti + 8 * (r >> 2) + lrow4 + (r & 3);
                                const int j = wn + 32 * tj + lcol;
                                T32[t32(i, j)] = acc[ti][tj][r];
                            }
                }
                __syncthreads();
#pragma clang loop unroll(disable)
                for (int idx = tid; idx < kHalf * (kBN / 4); idx += kNsThreads) {
                    const int rr = idx / (kBN / 4), c = (idx % (kBN / 4)) * 4;
                    const int64_t nr = row0 + h * kHalf + rr, nc = col0 + c;
                    if (nr >= g.R || nc >= g.Cn)
                        continue;
                    const f32x4_t o = *reinterpret_cast<const f32x4_t*>(T32 + t32(rr, c));
                    const int64_t base = nr * g.Cn + nc;
                    if (vec) {   /* nc + 3 < Cn: Cn and nc are multiples of 4 */
                        if constexpr (EPI == kEpiUpdate) {
                            f32x4_t w = *reinterpret_cast<const f32x4_t*>(W + base);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x = w[e] * k1;   /* decoupled decay first ([HANDBOOK] listing) */
                                const float u = k2 * o[e];
                                w[e] = x - u;
                            }
                            *reinterpret_cast<f32x4_t*>(W + base) = w;
                            if (Pm != nullptr) {
                                u32x2_t pb;
                                pb.x = bf16_rne_bits(w[0]) | (bf16_rne_bits(w[1]) << 16);
                                pb.y = bf16_rne_bits(w[2]) | (bf16_rne_bits(w[3]) << 16);
                                *reinterpret_cast<u32x2_t*>(Pm + base) = pb;
                            }
                        } else {
                            *reinterpret_cast<f32x4_t*>(g.out + base) = o;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (nc + e >= g.Cn)
                                break;
                            if constexpr (EPI == kEpiUpdate) {
                                float w = W[base + e] * k1;
                                const float u = k2 * o[e];
                                w = w - u;
                                W[base + e] = w;
                                if (Pm != nullptr)
                                    Pm[base + e] = static_cast<uint16_t>(bf16_rne_bits(w));
                            } else {
                                g.out[base + e] = o[e];
                            }
                        }
                    }
                }
            }
        }
    }
}

template <typename... Args>
hipError_t launch3(void (*kernel)(Args...), dim3 grid, int block, hipStream_t stream, Args... args)
{
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(block), argv, 0, stream);
}

struct Dims {
    int64_t mp, np;
};

/* One NS step's three GEMMs on a batch. */
/* Runs one launch between the hook's before / after calls. */
template <typename F>
hipError_t hooked(const NsHook* hook, int kind, double flops, F&& launch_fn)
{
    if (hook)
        hook->fn(hook->ctx, kind, 0, flops);
    hipError_t e = launch_fn();
    if (hook && e == hipSuccess)
        hook->fn(hook->ctx, kind, 1, flops);
    return e;
}

hipError_t ns_step(const TensorDesc* d_desc, const MuonInfo* d_info, const MuonBatch& b, const MuonWork& w,
                   const MuonGate& gate, float a, float bc, float cc, int cur, bool last, const MuonUpdate& up,
                   float* out, hipStream_t stream, const NsHook* hook)
{
    const double cntd = static_cast<double>(b.count), md = static_cast<double>(b.m), nd = static_cast<double>(b.n);
    const double f_gram = cntd * md * (md + 1.0) * nd;
    const double f_poly = cntd * md * md * (md + 1.0);
    const double f_step = cntd * 2.0 * md * md * nd;
    const int64_t mp = b.mp, np = b.np;
    const uint32_t cnt = static_cast<uint32_t>(b.count);
    GemmArgs g{};
    g.gate = gate;
    g.first = b.first;
    g.desc = d_desc;
    g.info = d_info;
    /* A = X X^T */
    g.P = w.X; g.ldp = np; g.sp = mp * np;
    g.Q = w.X; g.ldq = np; g.sq = mp * np;
    g.K = static_cast<int32_t>(np);
    g.C = w.A; g.ldc = mp; g.sc = mp * mp;
    const int32_t nt = static_cast<int32_t>(mp / SymTile::kBM);
    const dim3 tri(static_cast<uint32_t>(nt * (nt + 1) / 2), 1, cnt);
    g.nt = nt;
    hipError_t e = hooked(hook, HPO_MUON_PROF_GRAM, f_gram,
                          [&] { return launch3(k_ns_gemm<kEpiGram, true, SymTile>, tri, SymTile::kThreads, stream, g, up); });
    if (e != hipSuccess)
        return e;
    /* B = b A + c A A^T */
    g.P = w.A; g.ldp = mp; g.sp = mp * mp;
    g.Q = w.A; g.ldq = mp; g.sq = mp * mp;
    g.K = static_cast<int32_t>(mp);
    g.C = w.B; g.ldc = mp; g.sc = mp * mp;
    g.b = bc; g.c = cc;
    e = hooked(hook, HPO_MUON_PROF_POLY, f_poly,
               [&] { return launch3(k_ns_gemm<kEpiPoly, true, SymTile>, tri, SymTile::kThreads, stream, g, up); });
    if (e != hipSuccess)
        return e;
    /* X' = a X + B X  (Q = X^T, rows of X^T are columns of X) */
    g.P = w.B; g.ldp = mp; g.sp = mp * mp;
    g.Q = w.XT[cur]; g.ldq = mp; g.sq = np * mp;
    g.K = static_cast<int32_t>(mp);
    g.X = w.X; g.ldx = np; g.sx = mp * np;
    g.XT = w.XT[cur ^ 1]; g.ldxt = mp; g.sxt = np * mp;
    g.XS = w.XT[cur]; g.ldxs = mp; g.sxs = np * mp;
    g.a = a;
    g.nx = static_cast<int32_t>(np / GenTile::kBN);
    g.ny = static_cast<int32_t>(mp / GenTile::kBM);
    dim3 grid(static_cast<uint32_t>(g.nx * g.ny), 1, cnt);
    if (!last)
        return hooked(hook, HPO_MUON_PROF_STEP, f_step,
                      [&] { return launch3(k_ns_gemm<kEpiStep, false, GenTile>, grid, GenTile::kThreads, stream, g, up); });
    g.R = b.m;
    g.Cn = b.n;
    if (b.transposed) {
        /* The natural orientation is the transpose: compute O^T = a X^T + X^T B
         * (B is symmetric) as C = X^T B^T, so the output tile comes out in
         * the master's own row-major order and the update's reads and writes
         * of W run along its rows. */
        g.P = w.XT[cur]; g.ldp = mp; g.sp = np * mp;
        g.Q = w.B; g.ldq = mp; g.sq = mp * mp;
        g.X = w.XT[cur]; g.ldx = mp; g.sx = np * mp;
        g.XS = w.X; g.ldxs = np; g.sxs = mp * np;
        g.nx = static_cast<int32_t>(mp / GenTile::kBN);
        g.ny = static_cast<int32_t>(np / GenTile::kBM);
        grid.x = static_cast<uint32_t>(g.nx * g.ny);   /* tiles need not be square */
        g.R = b.n;
        g.Cn = b.m;
    }
    if (out != nullptr) {
        g.out = out;
        return hooked(hook, HPO_MUON_PROF_UPDATE, f_step,
                      [&] { return launch3(k_ns_gemm<kEpiOut, false, GenTile>, grid, GenTile::kThreads, stream, g, up); });
    }
    return hooked(hook, HPO_MUON_PROF_UPDATE, f_step,
                  [&] { return launch3(k_ns_gemm<kEpiUpdate, false, GenTile>, grid, GenTile::kThreads, stream, g, up); });
}

}  // namespace

hipError_t launch_muon_momentum(const SetView& sv, const MuonInfo* d_info, const MuonBatch& b, const MuonScalars& sc,
                                const MuonWork& w, hipStream_t stream)
{
    const int64_t n = b.c1 - b.c0;
    if (n > 0) {
        hipError_t e;
        const int64_t stride = b.gt_stride;
        if (sc.form == HPO_MUON_MOMENTUM_SUM)
            e = sc.nesterov ? launch3(k_muon_momentum<HPO_MUON_MOMENTUM_SUM, true>, dim3(n), kBlock, stream, sv, sc, b,
                                      w.gt, stride, w.part)
                            : launch3(k_muon_momentum<HPO_MUON_MOMENTUM_SUM, false>, dim3(n), kBlock, stream, sv, sc,
                                      b, w.gt, stride, w.part);
        else
            e = sc.nesterov ? launch3(k_muon_momentum<HPO_MUON_MOMENTUM_EMA, true>, dim3(n), kBlock, stream, sv, sc, b,
                                      w.gt, stride, w.part)
                            : launch3(k_muon_momentum<HPO_MUON_MOMENTUM_EMA, false>, dim3(n), kBlock, stream, sv, sc,
                                      b, w.gt, stride, w.part);
        if (e != hipSuccess)
            return e;
    }
    return launch3(k_muon_norm, dim3(static_cast<uint32_t>(b.count)), kBlock, stream, d_info, sc.gate, b.first,
                   static_cast<const double*>(w.part), sc.eps, w.dnorm);
}

hipError_t launch_muon_ns_input(const MuonBatch& b, const MuonWork& w, const MuonGate& gate, hipStream_t stream)
{
    const int64_t R = b.transposed ? b.n : b.m;
    const int64_t C = b.transposed ? b.m : b.n;
    const int64_t Rp = b.transposed ? b.np : b.mp;
    const int64_t Cp = b.transposed ? b.mp : b.np;
    uint16_t* copy = b.transposed ? w.XT[0] : w.X;
    uint16_t* trans = b.transposed ? w.X : w.XT[0];
    const int64_t ld_copy = b.transposed ? b.mp : b.np;
    const int64_t ld_trans = b.transposed ? b.np : b.mp;
    const int64_t s = b.mp * b.np;
    const dim3 grid(static_cast<uint32_t>(Cp / kTile), static_cast<uint32_t>(Rp / kTile),
                    static_cast<uint32_t>(b.count));
    return launch3(k_muon_ns_input, grid, kBlock, stream, static_cast<const float*>(w.gt), b.gt_stride,
                   static_cast<const float*>(w.dnorm), b.first, R, C, copy, ld_copy, s, trans, ld_trans, s, gate);
}

hipError_t launch_ns_input_from(const float* G, float eps, const MuonBatch& b, const MuonWork& w, hipStream_t stream)
{
    const int64_t n = b.m * b.n;
    constexpr int64_t kPer = 1 << 16;
    const int64_t blocks = n > 0 ? (n + kPer - 1) / kPer : 1;
    hipError_t e = launch3(k_sumsq_rows, dim3(static_cast<uint32_t>(blocks)), kBlock, stream, G, n, kPer, w.part);
    if (e != hipSuccess)
        return e;
    e = launch3(k_sumsq_fold, dim3(1), kBlock, stream, static_cast<const double*>(w.part),
                static_cast<int32_t>(blocks), eps, w.dnorm);
    if (e != hipSuccess)
        return e;
    MuonWork w2 = w;
    w2.gt = const_cast<float*>(G);
    MuonGate open{};
    return launch_muon_ns_input(b, w2, open, stream);
}

hipError_t launch_muon_ns(const TensorDesc* d_desc, const MuonInfo* d_info, const MuonBatch& b, const MuonWork& w,
                          const MuonGate& gate, int32_t steps, const float* coeffs, const MuonUpdate& up, float* out,
                          hipStream_t stream, const NsHook* hook)
{
    int cur = 0;
    for (int32_t s = 0; s < steps; ++s) {
        const bool last = s + 1 == steps;
        hipError_t e = ns_step(d_desc, d_info, b, w, gate, coeffs[3 * s], coeffs[3 * s + 1], coeffs[3 * s + 2], cur,
                               last, up, out, stream, hook);
        if (e != hipSuccess)
            return e;
        cur ^= 1;
    }
    return hipSuccess;
}

}  // namespace hpo
