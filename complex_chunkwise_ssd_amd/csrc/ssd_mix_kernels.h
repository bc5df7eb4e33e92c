// ssd_mix_kernels.h -- the MIMO head mixer that follows the scan (index.html
// lab 02 "MIMO MIXER": a fully connected mixer across the SSM heads, identity
// at initialisation; the AGENTS page, "Knows cold" item 2). One H x H real
// matrix W mixes the heads of every token, the same for every head-dim channel:
//     z[m, i, d] = sum_j W[i, j] y[m, j, d]           (m = token, i, j = heads)
// and, for a loss with upstream gradient gz,
//     gy[m, j, d] = sum_i W[i, j] gz[m, i, d]           (the mixer with W^T)
//     gW[i, j]    = sum_{m, d} gz[m, i, d] y[m, j, d]
//
// The mix itself moves 8 bytes per element for 2H flops: it is bound by HBM,
// so it runs on the vector ALUs with every token row read and written once,
// coalesced. gW is a genuine contraction over all M*D (token, channel) pairs
// into a 16 x 16 tile per pair of head blocks, so it runs on fp32 MFMA: each
// wave accumulates its tokens' outer products in four accumulator registers
// per tile, and a second small kernel adds the per-workgroup tiles in a fixed
// order (bit-identical results from run to run).
#pragma once

#include <ssd_device.h>

namespace ssd {

constexpr int kMixThreads = 256;    // four wave64s
constexpr int kMixMaxH = 32;        // heads the mixer kernels support
constexpr int kMixGwGroups = 1024;  // most workgroups (partial gW tiles) of the gW pass
constexpr int kMixUB = 4;           // channel groups of one gW load batch

struct MixParams {
    const float *in;  // (M, H, D)
    const float *W;   // (H, H) row-major
    float *out;       // (M, H, D); may be `in` itself (each thread reads a column before writing it)
    int64_t M;        // tokens
    int H, D;
    int transpose;    // 0: out_i = sum_j W[i][j] in_j    1: out_i = sum_j W[j][i] in_j
};

struct MixGradParams {
    const float *y;    // (M, H, D) mixer input of the forward
    const float *gz;   // (M, H, D) upstream gradient of the mixer output
    float *partial;    // (gridDim.x, H, H) one gW tile set per workgroup
    int64_t M;
    int H, D;
    const float *W;    // (H, H): the fused pass also forms grad_y
    float *gy;         // (M, H, D)
};

constexpr int kMixCB = 64;            // channels of one staged token tile in the fused pass
constexpr int kMixLd = kMixCB + 4;    // its row stride (floats) in shared memory

template <int DV>
struct MixVec;
template <>
struct MixVec<4> {
    typedef v4f T;
    static SSD_DEVICE T zero() { return v4f{0.f, 0.f, 0.f, 0.f}; }
    static SSD_DEVICE T load(const float *p) { return *(const v4f *)p; }
    static SSD_DEVICE T load(buf_t r, uint32_t off) { return buf_load4(r, off); }
    static SSD_DEVICE void store(float *p, T v) { *(v4f *)p = v; }
    static SSD_DEVICE float at(T v, int c) { return v[c]; }
};
template <>
struct MixVec<1> {
    typedef float T;
    static SSD_DEVICE T zero() { return 0.f; }
    static SSD_DEVICE T load(const float *p) { return *p; }
    static SSD_DEVICE T load(buf_t r, uint32_t off) { return buf_load1(r, off); }
    static SSD_DEVICE void store(float *p, T v) { *p = v; }
    static SSD_DEVICE float at(T v, int) { return v; }
};

// One thread per (token, group of DV head-dim channels): it reads that column
// of all H heads (consecutive threads read consecutive channels of one head
// row, so each head row of a token is one contiguous run), forms every output
// head from the weights in shared memory and writes the column back.
// DV = 4 needs D % 4 == 0 and 16-byte aligned rows.
template <int HMAX, int DV>
SSD_KERNEL(kMixThreads) void mix_kernel(MixParams p)
{
    typedef MixVec<DV> V;
    typedef typename V::T VT;
    SSD_LDS float sW[HMAX * HMAX];  // sW[i * HMAX + j]: weight of input head j in output head i
    const int tid = thread_id();
    for (int e = tid; e < HMAX * HMAX; e += kMixThreads) {
        const int i = e / HMAX, j = e % HMAX;
        float w = 0.f;
        if (i < p.H && j < p.H)
            w = p.transpose ? p.W[j * p.H + i] : p.W[i * p.H + j];
        sW[e] = w;
    }
    block_sync();
    const int G = p.D / DV;
    const int64_t HD = (int64_t)p.H * p.D;
    const int64_t cols = p.M * G;
    const int64_t stride = grid_blocks() * kMixThreads;
    for (int64_t c = block_id() * kMixThreads + tid; c < cols; c += stride) {
        const int64_t m = c / G;
        const int64_t base = m * HD + (int64_t)(c - m * G) * DV;
        // heads past H re-read the last head; their weights are zero
        VT v[HMAX];
#pragma unroll
        for (int j = 0; j < HMAX; ++j)
            v[j] = V::load(p.in + base + (int64_t)(j < p.H ? j : p.H - 1) * p.D);
#pragma unroll
        for (int i = 0; i < HMAX; ++i) {
            if (i >= p.H)
                break;
            VT acc = V::zero();
#pragma unroll
            for (int j = 0; j < HMAX; ++j)
                acc += sW[i * HMAX + j] * v[j];
            V::store(p.out + base + (int64_t)i * p.D, acc);
        }
    }
}

// gW partial tiles. The head blocks are 16 wide (HT of them); wave w of
// workgroup b takes tokens m = 4b + w, 4b + w + 4*grid, ... For one token, lane
// L = (r = L % 16, q = L / 16) reads DV channels of head 16a + r at channel
// d0 = 4*DV*u + DV*q of gz (the MFMA's A operand, row = output head i) and of
// y (its B operand, column = input head j); the four q lanes supply the four
// k values of one 16x16x4 step, so every (token, channel) pair is one k of the
// contraction. Heads past H and channels past D enter as zeros.
template <int HT, int DV>
SSD_KERNEL(kMixThreads) void mix_gw_kernel(MixGradParams p)
{
    typedef MixVec<DV> V;
    typedef typename V::T VT;
    constexpr int HP = 16 * HT;
    SSD_LDS float sPart[4][HP * HP];
    const int tid = thread_id();
    const int wave = wave_id();
    const int lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t HD = (int64_t)p.H * p.D;
    const int KG = (p.D + 4 * DV - 1) / (4 * DV);
    v4f acc[HT][HT];
#pragma unroll
    for (int a = 0; a < HT; ++a)
#pragma unroll
        for (int b = 0; b < HT; ++b)
            acc[a][b] = MixVec<4>::zero();
    const int64_t wstride = grid_blocks() * 4;
    const uint32_t row_bytes = (uint32_t)(HD * 4);
    for (int64_t m = block_id() * 4 + wave; m < p.M; m += wstride) {
        // one token's rows; an offset at the end of the row reads zeros
        const buf_t gzm = make_buf(p.gz + m * HD, row_bytes);
        const buf_t ym = make_buf(p.y + m * HD, row_bytes);
        // UB channel groups are loaded together (all loads in flight at once),
        // then contracted; channels past D read zeros
        for (int u0 = 0; u0 < KG; u0 += kMixUB) {
            VT g[kMixUB][HT], v[kMixUB][HT];
#pragma unroll
            for (int uu = 0; uu < kMixUB; ++uu) {
                const int d0 = 4 * DV * (u0 + uu) + DV * q;
#pragma unroll
                for (int a = 0; a < HT; ++a) {
                    const int h = 16 * a + r;
                    const uint32_t off =
                        (h < p.H && d0 < p.D) ? (uint32_t)(h * p.D + d0) * 4 : row_bytes;
                    g[uu][a] = V::load(gzm, off);
                    v[uu][a] = V::load(ym, off);
                }
            }
            sched_fence();  // issue every load of the batch before the first MFMA
#pragma unroll
            for (int uu = 0; uu < kMixUB; ++uu)
#pragma unroll
                for (int c = 0; c < DV; ++c)
#pragma unroll
                    for (int a = 0; a < HT; ++a)
#pragma unroll
                        for (int b = 0; b < HT; ++b)
                            acc[a][b] = mfma_16x16x4(V::at(g[uu][a], c), V::at(v[uu][b], c),
                                                     acc[a][b]);
        }
    }
    // lane L holds rows 4q..4q+3 of column r of each tile
#pragma unroll
    for (int a = 0; a < HT; ++a)
#pragma unroll
        for (int b = 0; b < HT; ++b)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                sPart[wave][(16 * a + 4 * q + k) * HP + 16 * b + r] = acc[a][b][k];
    block_sync();
    float *dst = p.partial + block_id() * (int64_t)p.H * p.H;
    for (int e = tid; e < p.H * p.H; e += kMixThreads) {
        const int i = e / p.H, j = e % p.H;
        const int o = i * HP + j;
        dst[e] = ((sPart[0][o] + sPart[1][o]) + sPart[2][o]) + sPart[3][o];
    }
}

// The fused backward for H <= 16 and D % 4 == 0 (16-byte aligned rows): one
// pass over grad_z and y forms both grad_y and the gW partial tiles, so grad_z
// is read once. Each wave takes whole tokens (4b + w, then every 4*grid); per
// token and 64-channel block it loads the 16 x 64 tiles of grad_z and y with
// row-contiguous 16-byte loads (lane l covers floats 4l + 256k of the tile),
// issued one token ahead, and stages them in its own shared-memory tiles. From
// there: the gW tile on MFMA exactly as in mix_gw_kernel (lane (r, q) reads
// head r, channels 16u + 4q ..), and grad_y on the vector ALUs: lane (g, s)
// forms output heads 4s .. 4s+3 at channels 4g .. 4g+3 from all 16 input
// heads, reading W[i][4s .. 4s+3] from shared memory (a broadcast read).
SSD_KERNEL(kMixThreads) void mix_bwd_fused_kernel(MixGradParams p)
{
    SSD_LDS float sG[4][16 * kMixLd];
    SSD_LDS float sY[4][16 * kMixLd];
    SSD_LDS float sPart[4][16 * 16];
    SSD_LDS float sW[16 * 16];  // sW[i * 16 + j] = W[i][j], zero past H
    const int tid = thread_id();
    const int wave = wave_id();
    const int lane = tid & 63;
    const int r = lane & 15, q = lane >> 4;  // MFMA roles; also (g, s) of grad_y
    const int64_t HD = (int64_t)p.H * p.D;
    const uint32_t row_bytes = (uint32_t)(HD * 4);
    const int nblk = (p.D + kMixCB - 1) / kMixCB;

    static_assert(kMixThreads == 16 * 16, "one thread per weight");
    {
        const int i = tid >> 4, j = tid & 15;
        sW[tid] = i < p.H && j < p.H ? p.W[i * p.H + j] : 0.f;
    }
    block_sync();

    // tile element f = 4 lane + 256 k (k < 4): head f / 64, channel f % 64 of the
    // block; heads past H and channels past D read zero
    auto tile_off = [&](int cb, int k) {
        const int f = 4 * lane + 256 * k, i = f >> 6, c = f & 63;
        const int d = kMixCB * cb + c;
        return i < p.H && d < p.D ? (uint32_t)(i * p.D + d) * 4 : row_bytes;
    };
    struct Tiles {
        v4f g[4], v[4];
    };
    auto fetch = [&](int64_t m, int cb, Tiles &t) {
        const bool live = m < p.M;
        const buf_t bg = make_buf(p.gz + (live ? m : 0) * HD, live ? row_bytes : 0u);
        const buf_t by = make_buf(p.y + (live ? m : 0) * HD, live ? row_bytes : 0u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t o = tile_off(cb, k);
            t.g[k] = buf_load4(bg, o);
            t.v[k] = buf_load4(by, o);
        }
    };

    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    const int64_t wstride = grid_blocks() * 4;
    int64_t m = block_id() * 4 + wave;
    int cb = 0;
    Tiles nx;
    fetch(m, cb, nx);
    float *tg = sG[wave];
    float *ty = sY[wave];
    while (m < p.M) {
        const Tiles cur = nx;
        const int64_t mc = m;
        const int cbc = cb;
        if (++cb == nblk) {
            cb = 0;
            m += wstride;
        }
        fetch(m, cb, nx);  // the next tile is in flight while this one is used
        wave_lds_sync();   // the previous tile's reads are done
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int f = 4 * lane + 256 * k, i = f >> 6, c = f & 63;
            *(v4f *)&tg[i * kMixLd + c] = cur.g[k];
            *(v4f *)&ty[i * kMixLd + c] = cur.v[k];
        }
        wave_lds_sync();
        // gW: head r of grad_z against head r of y at channels 16u + 4q + 0..3
#pragma unroll
        for (int u = 0; u < kMixCB / 16; ++u) {
            const v4f a4 = *(const v4f *)&tg[r * kMixLd + 16 * u + 4 * q];
            const v4f b4 = *(const v4f *)&ty[r * kMixLd + 16 * u + 4 * q];
            acc = mfma_16x16x4(a4.x, b4.x, acc);
            acc = mfma_16x16x4(a4.y, b4.y, acc);
            acc = mfma_16x16x4(a4.z, b4.z, acc);
            acc = mfma_16x16x4(a4.w, b4.w, acc);
        }
        // grad_y at output heads 4q + jj, channels 4r .. 4r + 3 of the block
        v4f o[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            o[jj] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const v4f gv = *(const v4f *)&tg[i * kMixLd + 4 * r];
            const v4f w4 = *(const v4f *)&sW[i * 16 + 4 * q];
            o[0] += w4.x * gv;
            o[1] += w4.y * gv;
            o[2] += w4.z * gv;
            o[3] += w4.w * gv;
        }
        const int d = kMixCB * cbc + 4 * r;
        float *gyrow = p.gy + mc * HD + d;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * q + jj;
            if (j < p.H && d < p.D)
                *(v4f *)(gyrow + (int64_t)j * p.D) = o[jj];
        }
    }
    // lane L holds rows 4q..4q+3 of column r of the wave's tile
#pragma unroll
    for (int k = 0; k < 4; ++k)
        sPart[wave][(4 * q + k) * 16 + r] = acc[k];
    block_sync();
    float *dst = p.partial + block_id() * (int64_t)p.H * p.H;
    for (int e = tid; e < p.H * p.H; e += kMixThreads) {
        const int o = (e / p.H) * 16 + e % p.H;
        dst[e] = ((sPart[0][o] + sPart[1][o]) + sPart[2][o]) + sPart[3][o];
    }
}

// gW[i][j] = the sum of the partial tiles, one wave64 per entry: lane l adds
// tiles l, l + 64, ... in double, and lane 0 adds the 64 lane sums in lane
// order (a fixed order, so the result does not vary from run to run).
SSD_KERNEL(64) void mix_gw_reduce_kernel(const float *partial, int groups, int HH, float *gW)
{
    SSD_LDS double sSum[64];
    const int e = (int)block_id();
    const int lane = thread_id();
    double s = 0.0;
#pragma unroll 8
    for (int g = lane; g < groups; g += 64)
        s += (double)partial[(int64_t)g * HH + e];
    sSum[lane] = s;
    block_sync();
    if (lane == 0) {
        double t = 0.0;
        for (int k = 0; k < 64; ++k)
            t += sSum[k];
        gW[e] = (float)t;
    }
}

}  // namespace ssd
