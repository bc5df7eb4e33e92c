// ssd_mix_kernels.h -- the MIMO head mixer that follows the scan, and its
// gradients, as fp32 MFMA matrix products.
//
// The mixer (index.html lab 02 "MIMO MIXER": 1024 -> 1024 as 16 heads of 64
// channels, fully connected across the heads, identity at initialisation; the
// model's parameter count in the "Extending" guide's documentation rule, which
// holds only with a dense 1024 x 1024 matrix per layer) maps the heads of each
// token, flattened head-major (k = h * D + d, F = H * D), by one dense real
// F x F matrix W (row o = the weights of output o):
//     z[m, o]  = sum_k W[o, k] y[m, k]          z  = y W^T
//     gy[m, k] = sum_o gz[m, o] W[o, k]         gy = gz W
//     gW[o, k] = sum_m gz[m, o] y[m, k]         gW = gz^T y
// Each costs 2 M F^2 flops for about 8 M F + 4 F^2 bytes -- near 500 flops per
// byte at F = 1024, far past the fp32 MFMA ridge of ~20 -- so all three run on
// one tiled fp32 MFMA 16x16x4 product, gemm_kernel, whose operand layouts are
// template arguments:
//     C[m, n] = sum_k A(m, k) B(n, k)
//     A(m, k) = a[m * lda + k]  (AT = false)   or  a[k * lda + m]  (AT = true)
//     B(n, k) = b[n * ldb + k]  (BT = false)   or  b[k * ldb + n]  (BT = true)
// z takes A = y, B = W; gy takes A = gz and B = W with BT; gW takes A = gz and
// B = y, both with AT/BT (its sum runs over the tokens), cut into token ranges
// ("splits") whose partial products split_sum_kernel adds in a fixed order.
//
// Tiling: a workgroup of 8 wave64s computes a 256 x 256 tile of C; wave w holds
// rows 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63 as 8 x 4 MFMA blocks
// (128 accumulator registers per lane). K advances 16 at a time through two
// shared-memory stages: while the waves multiply one 256 x 16 tile of A and B,
// each thread holds its share of the next tile in registers (loaded one tile
// ahead) and writes it to the other stage halfway through, so one workgroup
// barrier per 16-wide step orders everything.
//
// MFMA k order: in step s (0..3) of a 16-wide tile, the lanes with q = L / 16
// supply k = 4 q + s. A K-contiguous operand is staged as rows of 16 floats
// (stride 20), so a lane reads its four k with one 16-byte load; a
// row-contiguous (transposed) operand is staged as 16 rows of 256 (stride 260)
// and read one float per step. Both strides keep the reads free of bank
// conflicts.
#pragma once

#include <ssd_device.h>

namespace ssd {

constexpr int kGemmThreads = 512;          // 8 wave64s: 2 (rows) x 4 (columns)
constexpr int kGemmBM = 256;               // rows of C per workgroup
constexpr int kGemmBN = 256;               // columns of C per workgroup
constexpr int kGemmBK = 16;                // K of one staged tile (4 MFMA steps)
constexpr int kGemmLdK = kGemmBK + 4;      // row stride of a K-contiguous staged tile
constexpr int kGemmLdT = kGemmBM + 4;      // row stride of a transposed staged tile
constexpr int kGemmStage = kGemmBM * kGemmLdK;  // floats per stage (>= kGemmBK * kGemmLdT)
constexpr uint32_t kGemmOut = 0x80000000u;      // a byte offset past every buffer
constexpr int kMixMaxF = 16384;                 // largest H * D the mixer takes
constexpr int kMixMinSplitTokens = 1024;        // fewest tokens per gW split
constexpr int kMixMaxWorkgroups = 256;          // gW splits aim at one workgroup per CU

static_assert(kGemmBK * kGemmLdT <= kGemmStage, "stage too small for a transposed tile");

struct GemmParams {
    const float *a;
    const float *b;
    float *c;
    int64_t lda, ldb, ldc;
    int64_t c_split;  // floats between the C blocks of two K splits
    int M, N, K;
    int tiles_m, tiles_n, splits;
    int kchunk;       // K per split, a multiple of kGemmBK
};

// One thread's share of a staged 256 x 16 operand tile: two groups of four
// floats. K-contiguous (TR = false): group f = tid + 512 g is row f / 4,
// k = k0 + 4 (f % 4) .. +3; the buffer starts at row r0 and holds `rows` rows
// (fewer at the edge of the matrix), and k at or past kend reads zero.
// Transposed (TR = true): group f is k row k0 + f / 64, rows r0 + 4 (f % 64)
// .. +3; the buffer holds the k rows below kend, and rows at or past `extent`
// read zero. VEC = false loads each float on its own (any alignment).
template <bool TR, bool VEC>
SSD_DEVICE void gemm_stage_load(v4f (&g)[2], const float *x, int64_t ld, int r0, int extent,
                                int k0, int kend, int tid)
{
    if (!TR) {
        const int rows = extent - r0 < kGemmBM ? extent - r0 : kGemmBM;
        const buf_t rs = make_buf(x + (int64_t)r0 * ld, (uint32_t)(rows * ld * 4));
        for (int gi = 0; gi < 2; ++gi) {
            const int f = tid + kGemmThreads * gi;
            const int r = f >> 2, k = k0 + 4 * (f & 3);
            const uint32_t base = (uint32_t)(r * ld + k) * 4u;
            if (VEC) {
                g[gi] = buf_load4(rs, k < kend ? base : kGemmOut);
            } else {
                for (int e = 0; e < 4; ++e)
                    g[gi][e] = buf_load1(rs, k + e < kend ? base + 4u * e : kGemmOut);
            }
        }
    } else {
        int krows = kend - k0;
        krows = krows < 0 ? 0 : (krows > kGemmBK ? kGemmBK : krows);
        const buf_t rs = make_buf(x + (int64_t)k0 * ld + r0, (uint32_t)(krows * ld * 4));
        for (int gi = 0; gi < 2; ++gi) {
            const int f = tid + kGemmThreads * gi;
            const int kr = f >> 6, c = 4 * (f & 63);
            const uint32_t base = (uint32_t)(kr * ld + c) * 4u;
            if (VEC) {
                g[gi] = buf_load4(rs, r0 + c < extent ? base : kGemmOut);
            } else {
                for (int e = 0; e < 4; ++e)
                    g[gi][e] = buf_load1(rs, r0 + c + e < extent ? base + 4u * e : kGemmOut);
            }
        }
    }
}

template <bool TR>
SSD_DEVICE void gemm_stage_store(float *s, const v4f (&g)[2], int tid)
{
    for (int gi = 0; gi < 2; ++gi) {
        const int f = tid + kGemmThreads * gi;
        if (!TR)
            *(v4f *)&s[(f >> 2) * kGemmLdK + 4 * (f & 3)] = g[gi];
        else
            *(v4f *)&s[(f >> 6) * kGemmLdT + 4 * (f & 63)] = g[gi];
    }
}

// The four k (4 q + s, s = 0..3) of staged row `row` that lane group q supplies.
template <bool TR>
SSD_DEVICE v4f gemm_operand(const float *s, int row, int q)
{
    if (!TR)
        return *(const v4f *)&s[row * kGemmLdK + 4 * q];
    return v4f{s[(4 * q + 0) * kGemmLdT + row], s[(4 * q + 1) * kGemmLdT + row],
               s[(4 * q + 2) * kGemmLdT + row], s[(4 * q + 3) * kGemmLdT + row]};
}

template <bool AT, bool BT, bool VEC>
SSD_KERNEL(kGemmThreads) void gemm_kernel(GemmParams p)
{
    SSD_LDS float sA[2 * kGemmStage];
    SSD_LDS float sB[2 * kGemmStage];
    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int wm = w >> 2, wn = w & 3;
    const int l16 = lane & 15, q = lane >> 4;

    // Workgroup -> (split, row tile, column tile). The workgroups that share a
    // block of A rows (one split and row tile) go to one XCD when the number of
    // such blocks allows it (workgroup i runs on XCD i % 8), so that the XCD's L2
    // serves their A loads.
    const int64_t id = block_id();
    const int units = p.splits * p.tiles_m;
    int unit, tn;
    if (units % 8 == 0) {
        const int64_t slot = id >> 3;
        unit = (int)((slot / p.tiles_n) * 8 + (id & 7));
        tn = (int)(slot % p.tiles_n);
    } else {
        unit = (int)(id / p.tiles_n);
        tn = (int)(id % p.tiles_n);
    }
    const int split = unit / p.tiles_m, tm = unit % p.tiles_m;
    const int m0 = tm * kGemmBM, n0 = tn * kGemmBN;
    const int kb = split * p.kchunk;
    const int ke = p.K < kb + p.kchunk ? p.K : kb + p.kchunk;
    const int nkt = ke > kb ? (ke - kb + kGemmBK - 1) / kGemmBK : 0;

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v4f ga[2], gb[2];
    gemm_stage_load<AT, VEC>(ga, p.a, p.lda, m0, p.M, kb, ke, tid);
    gemm_stage_load<BT, VEC>(gb, p.b, p.ldb, n0, p.N, kb, ke, tid);
    gemm_stage_store<AT>(sA, ga, tid);
    gemm_stage_store<BT>(sB, gb, tid);
    gemm_stage_load<AT, VEC>(ga, p.a, p.lda, m0, p.M, kb + kGemmBK, ke, tid);
    gemm_stage_load<BT, VEC>(gb, p.b, p.ldb, n0, p.N, kb + kGemmBK, ke, tid);
    block_sync();

    const int arow = wm * 128 + l16, bcol = wn * 64 + l16;
    for (int kt = 0; kt < nkt; ++kt) {
        const float *cA = sA + (kt & 1) * kGemmStage;
        const float *cB = sB + (kt & 1) * kGemmStage;
        v4f bv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bv[j] = gemm_operand<BT>(cB, bcol + 16 * j, q);
        v4f av = gemm_operand<AT>(cA, arow, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const v4f a_cur = av;
            if (i + 1 < 8)
                av = gemm_operand<AT>(cA, arow + 16 * (i + 1), q);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma_16x16x4(a_cur[s], bv[j][s], acc[i][j]);
            if (i == 3) {
                // The other stage was last read before the previous barrier:
                // write the next tile there and start loading the one after.
                // Past the end of K the loads read zeros and the stage written
                // is never read.
                float *nA = sA + ((kt + 1) & 1) * kGemmStage;
                float *nB = sB + ((kt + 1) & 1) * kGemmStage;
                gemm_stage_store<AT>(nA, ga, tid);
                gemm_stage_store<BT>(nB, gb, tid);
                const int k2 = kb + (kt + 2) * kGemmBK;
                gemm_stage_load<AT, VEC>(ga, p.a, p.lda, m0, p.M, k2, ke, tid);
                gemm_stage_load<BT, VEC>(gb, p.b, p.ldb, n0, p.N, k2, ke, tid);
            }
        }
        block_sync();
    }

    // Lane (l16, q) holds C[16 i + 4 q + r][16 j + l16] of the wave's blocks.
    const int rows = p.M - m0 < kGemmBM ? p.M - m0 : kGemmBM;
    const buf_t cs = make_buf(p.c + split * p.c_split + (int64_t)m0 * p.ldc + n0,
                              (uint32_t)(rows * p.ldc * 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = wn * 64 + 16 * j + l16;
        const bool cin = n0 + col < p.N;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 128 + 16 * i + 4 * q + r;
                buf_store1(cs, cin ? (uint32_t)(row * p.ldc + col) * 4u : kGemmOut, acc[i][j][r]);
            }
    }
}

// out[e] = sum over s of part[s * stride + e], s in increasing order.
SSD_KERNEL(256) void split_sum_kernel(const float *part, int64_t stride, int splits, int64_t n,
                                      float *out)
{
    const int64_t step = grid_blocks() * 256;
    for (int64_t e = block_id() * 256 + thread_id(); e < n; e += step) {
        float acc = 0.f;
        for (int s = 0; s < splits; ++s)
            acc += part[s * stride + e];
        out[e] = acc;
    }
}

SSD_KERNEL(256) void fill_zero_kernel(float *out, int64_t n)
{
    const int64_t step = grid_blocks() * 256;
    for (int64_t e = block_id() * 256 + thread_id(); e < n; e += step)
        out[e] = 0.f;
}

}  // namespace ssd
