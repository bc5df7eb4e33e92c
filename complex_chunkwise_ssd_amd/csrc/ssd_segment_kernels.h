// ssd_segment_kernels.h -- the passes that join sequence segments after the scan
// has run them side by side (segment 0 from the initial state, the others from
// zero). This is the inter-chunk state passing of index.html lab 03 ("STATE"
// line: each chunk's state carried to the next with the chunk's total decay)
// applied once more at the coarser grain of segments, and the state-to-output
// term of the same lab applied to the state entering each segment:
//
//   prefix: H_in[1] = S_0, H_in[p+1] = exp(lam_p) H_in[p] + S_p, final = H_in[P]
//           (S_p: segment p's end state from its own start, lam_p its total
//           log-decay);
//   fix-up: for every token t of a segment p >= 1,
//           y_t += Re( exp(Lambda_t) C_t H_in[p] ),
//           Lambda_t = sum of softplus(dt) A from the segment start through t.
//
// The scan is linear in the state it starts from, so the two together give
// exactly the outputs and final state of one walk over the whole sequence.
#pragma once

#include <ssd_kernels.h>

namespace ssd {

// One thread per complex state element (b, h, n, d); the P segment states of
// the sequence are walked in order. Slot p-1 of seg_state receives H_in[p]
// (S_{p-1} has been read by then); the final state goes to final_state.
SSD_KERNEL(256) void segment_prefix_kernel(ScanParams p)
{
    const int64_t nd = (int64_t)p.N * p.D;
    const int64_t e = block_id() * 256 + thread_id();
    if (e >= (int64_t)p.B * p.H * nd)
        return;
    const int64_t bh = e / nd, k = e - bh * nd;
    float *slot = p.seg_state + (bh * p.P * nd + k) * 2;
    v2f hs = *(const v2f *)slot;
    // eight segments' states are read before any of their slots is written (one
    // memory round trip per eight segments)
    constexpr int QB = 8;
    for (int q0 = 1; q0 < p.P; q0 += QB) {
        v2f sq[QB], lg[QB];
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            sq[j] = lg[j] = v2f{0.f, 0.f};
            if (q0 + j < p.P) {  // the same for every thread
                sq[j] = *(const v2f *)(slot + (q0 + j) * nd * 2);
                lg[j] = *(const v2f *)&p.seg_logdecay[(bh * p.P + q0 + j) * 2];
            }
        }
        v2f ef[QB];
#pragma unroll
        for (int j = 0; j < QB; ++j)
            ef[j] = cexp_f(lg[j]);
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            if (q0 + j < p.P) {
                *(v2f *)(slot + (q0 + j - 1) * nd * 2) = hs;
                hs = cmul(ef[j], hs) + sq[j];
            }
        }
    }
    if (p.final_state)
        *(v2f *)&p.final_state[(bh * nd + k) * 2] = hs;
}

// The state-to-output term of a later segment's entering state. Workgroup =
// (sequence, segment p >= 1, 64-wide slice of D, group of the segment's
// chunks); wave w owns the 16 columns 16w..16w+15 of the slice. Per chunk, as
// a real fp32 MFMA product with K = 2N:
//   Re(C' H) = [Re C' | -Im C'] [Re H ; Im H],  C' = exp(Lambda_t) C_t,
// with H (the wave's columns) held in registers for the whole group and C'
// staged in shared memory by all threads, in two buffers taken in turn: one
// barrier per chunk. Every wave takes the chunk's decays itself. Step s = 4u + j
// of the 32 K-steps uses k = 16u + 4 (L / 16) + j on lane L, so each lane reads
// its four A values of four steps as one 16-byte word; the chunk's row tiles
// are independent accumulators, interleaved step by step.
template <int R, int LAYOUT>
SSD_KERNEL(kFixThreads) void segment_fixup_kernel(ScanParams p)
{
    constexpr bool PROJ = LAYOUT != kLayoutC64;
    constexpr bool BF16 = LAYOUT == kLayoutProjBf16;
    constexpr uint32_t ES = BF16 ? 2u : 4u;  // bytes per element of an in_proj row
    constexpr int NR = R / 16;
    constexpr int LDK = 2 * kNPad + 4;       // floats per staged row: [Re C' | -Im C'] + pad
    constexpr int KSTEPS = 2 * kNPad / 4;    // MFMA steps over K = 2N (padded)
    constexpr int ROWS_PER_PASS = kFixThreads / (kNPad / 2);  // C rows loaded per pass: 8
    constexpr uint32_t kOut = 0x80000000u;
    static_assert(R % ROWS_PER_PASS == 0, "row passes must tile the chunk");

    SSD_LDS float sCp[2][R * LDK];

    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int Lr = lane & 15;
    const int Lk = lane >> 4;

    int64_t blk = block_id();
    const int grp = (int)(blk % p.fix_groups);
    blk /= p.fix_groups;
    const int db = (int)(blk % p.ndb);
    blk /= p.ndb;
    const int seg = 1 + (int)(blk % (p.P - 1));
    blk /= p.P - 1;
    const int h = (int)(blk % p.H);
    const int b = (int)(blk / p.H);
    const int64_t bh = (int64_t)b * p.H + h;

    const int s_begin = seg * p.spc;
    const int s_end = s_begin + p.spc < p.nc ? s_begin + p.spc : p.nc;
    const int per = (s_end - s_begin + p.fix_groups - 1) / p.fix_groups;
    const int c_begin = s_begin + grp * per;
    const int c_end = c_begin + per < s_end ? c_begin + per : s_end;
    if (c_begin >= c_end)
        return;  // the whole workgroup leaves together

    const v2f Ah = v2f{uniform(p.A[2 * h]), uniform(p.A[2 * h + 1])};
    const int dsl = p.D - db * kDBlock;  // columns of D from this slice on
    const int dl = 16 * w + Lr;          // this lane's column in the slice
    const bool dvalid = dl < dsl;
    const int dcol = db * kDBlock + dl;

    // With N above 64 the state is taken in 64-row slices, one after another: the
    // term is a sum over n, so each slice's share is added to y in turn.
    for (int ns = 0; ns < p.nnb; ++ns) {
        const int n0 = ns * kNPad;
        const int nsl = p.N - n0 < kNPad ? p.N - n0 : kNPad;  // rows of this slice

        // B operand: the state entering the segment (slot seg - 1 after the prefix
        // pass), rows k of [Re H ; Im H] of this slice at this lane's column.
        float hb[KSTEPS];
        {
            const float *hin = p.seg_state + (bh * p.P + (seg - 1)) * (int64_t)p.N * p.D * 2;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int k = 16 * (s >> 2) + 4 * Lk + (s & 3);
                const int n = k < kNPad ? k : k - kNPad;
                hb[s] = n < nsl && dvalid
                            ? hin[((int64_t)(n0 + n) * p.D + dcol) * 2 + (k < kNPad ? 0 : 1)]
                            : 0.f;
            }
        }

        const uint32_t prow = (uint32_t)p.tok_stride * ES;                  // in_proj row bytes
        const uint32_t brow = PROJ ? prow : (uint32_t)(p.H * p.N) * 8u;     // C_t row bytes
        const uint32_t drow = PROJ ? prow : (uint32_t)p.H * 4u;             // dt row bytes
        const uint32_t yrow = (uint32_t)(p.H * p.D) * 4u;
        const uint32_t imoff = (uint32_t)(p.H * p.N) * ES;                  // PROJ: Im plane
        const int64_t bt0 = (int64_t)b * p.T;
        auto at = [&](const float *base, int64_t e) { return (const void *)((const char *)base + e * ES); };
        auto rows_of = [&](int c) { return p.Q < p.T - c * p.Q ? p.Q : p.T - c * p.Q; };

        // C rows: thread (row r0 + tid / 32 of each pass, complex pair ncol/2 .. +1)
        const int ncol = (tid & 31) * 2;
        const uint32_t offC = ncol < nsl ? (uint32_t)(tid >> 5) * brow + ncol * (PROJ ? ES : 8u) : kOut;
        const uint32_t offY = dvalid ? (uint32_t)(4 * Lk) * yrow + dl * 4u : kOut;

        // A chunk's inputs in registers: dt (lanes below R, every wave), C rows, and
        // the y values this lane will update. fetch(c) issues the loads for chunk c; past
        // the group's last chunk every buffer is empty, so the loads still issue
        // (the wait counters stay exact) and read zero.
        struct Inputs {
            float dt;
            v4f cv[R / ROWS_PER_PASS];
            float yv[NR][4];
        };
        auto ybuf = [&](int c) {
            const int64_t tok = bt0 + (int64_t)c * p.Q;
            return c < c_end ? make_buf(p.y + (tok * p.H + h) * (int64_t)p.D + db * kDBlock,
                                        (uint32_t)(rows_of(c) - 1) * yrow + (uint32_t)dsl * 4u)
                             : make_buf(p.y, 0u);
        };
        auto fetch = [&](int c, Inputs &in) {
            const bool live = c < c_end;
            const uint32_t rows = live ? (uint32_t)rows_of(c) : 1u;
            const int64_t tok = bt0 + (int64_t)(live ? c : c_begin) * p.Q;
            const void *dt0 = PROJ ? at(p.dt, tok * p.tok_stride + h) : (const void *)(p.dt + tok * p.H + h);
            const buf_t bT = make_buf(dt0, live ? (rows - 1) * drow + ES : 0u);
            const uint32_t od = lane < R ? (uint32_t)lane * drow : kOut;
            in.dt = BF16 ? bf16_lo(buf_load_u16(bT, od)) : buf_load1(bT, od);
            const void *c0 = PROJ ? at(p.Ct, tok * p.tok_stride + (int64_t)h * p.N + n0)
                                  : (const void *)(p.Ct + ((tok * p.H + h) * (int64_t)p.N + n0) * 2);
            const buf_t bC = make_buf(c0, live ? (rows - 1) * brow + (PROJ ? imoff : 0u) +
                                                     nsl * (PROJ ? ES : 8u)
                                               : 0u);
#pragma unroll
            for (int i = 0; i < R / ROWS_PER_PASS; ++i) {
                const uint32_t o = offC + (uint32_t)(ROWS_PER_PASS * i) * brow;
                if constexpr (BF16) {
                    const uint32_t re = buf_load_u32(bC, o), im = buf_load_u32(bC, o + imoff);
                    in.cv[i] = v4f{bf16_lo(re), bf16_lo(im), bf16_hi(re), bf16_hi(im)};
                } else if constexpr (PROJ) {
                    const v2f re = buf_load2(bC, o), im = buf_load2(bC, o + imoff);
                    in.cv[i] = v4f{re.x, im.x, re.y, im.y};
                } else {
                    in.cv[i] = buf_load4(bC, o);
                }
            }
            const buf_t bY = ybuf(c);
#pragma unroll
            for (int t = 0; t < NR; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    in.yv[t][r] = buf_load1(bY, offY + (uint32_t)(16 * t + r) * yrow);
        };

        Inputs nx;
        fetch(c_begin, nx);
        if (ns > 0)
            block_sync();  // every wave is done with the previous slice's last buffers
        for (int c = c_begin; c < c_end; ++c) {
            const Inputs cur = nx;
            const uint32_t rows = (uint32_t)rows_of(c);
            float *cp = sCp[(c - c_begin) & 1];
            // Lambda_t for the chunk's rows (lane t): a = softplus(dt) A summed in
            // 16-lane rows, then the earlier rows' totals and the chunk-start log.
            const float sp = softplus_f(cur.dt);
            const v2f a = (uint32_t)lane < rows ? v2f{Ah.x * sp, Ah.y * sp} : v2f{0.f, 0.f};
            v2f lam = a;
            lam += v2f{row_shr<1>(lam.x), row_shr<1>(lam.y)};
            lam += v2f{row_shr<2>(lam.x), row_shr<2>(lam.y)};
            lam += v2f{row_shr<4>(lam.x), row_shr<4>(lam.y)};
            lam += v2f{row_shr<8>(lam.x), row_shr<8>(lam.y)};
            // a scalar load: a vector load here would make the wave wait for its
            // last chunk's y stores as well (one wait counter covers both)
            v2f base = ld_c_uniform(p.chunk_log, bh * p.nc + c);
            for (int t = 0; t < NR - 1; ++t) {
                const v2f tt = v2f{lane_read(lam.x, 16 * t + 15), lane_read(lam.y, 16 * t + 15)};
                if ((lane >> 4) > t)
                    base += tt;
            }
            const v2f e = cexp_f(lam + base);
#pragma unroll
            for (int i = 0; i < R / ROWS_PER_PASS; ++i) {
                const int row = ROWS_PER_PASS * i + (tid >> 5);
                const v2f er = v2f{lane_fetch(e.x, row), lane_fetch(e.y, row)};
                const v2f a0 = cmul(er, v2f{cur.cv[i].x, cur.cv[i].y});
                const v2f a1 = cmul(er, v2f{cur.cv[i].z, cur.cv[i].w});
                *(v2f *)&cp[row * LDK + ncol] = v2f{a0.x, a1.x};
                *(v2f *)&cp[row * LDK + kNPad + ncol] = v2f{-a0.y, -a1.y};
            }
            block_sync();
            fetch(c + 1, nx);  // in flight during the products
            const buf_t bY = ybuf(c);
            v4f acc[NR];
#pragma unroll
            for (int t = 0; t < NR; ++t)
                acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KSTEPS / 4; ++u) {
                v4f a4[NR];
#pragma unroll
                for (int t = 0; t < NR; ++t)
                    a4[t] = *(const v4f *)(cp + (16 * t + Lr) * LDK + 4 * Lk + 16 * u);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int t = 0; t < NR; ++t)
                        acc[t] = mfma_16x16x4(a4[t][j], hb[4 * u + j], acc[t]);
            }
            // lane holds rows 16t + 4Lk + r of column dl
#pragma unroll
            for (int t = 0; t < NR; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    buf_store1(bY, offY + (uint32_t)(16 * t + r) * yrow, cur.yv[t][r] + acc[t][r]);
        }
    }  // slices of N
}

// y = the sum of the per-slice partial outputs (N above 64), slices in order.
SSD_KERNEL(256) void slice_sum_kernel(const float *part, int nnb, int64_t n, float *y)
{
    const int64_t stride = grid_blocks() * 256;
    for (int64_t e = block_id() * 256 + thread_id(); e < n; e += stride) {
        float s = part[e];
        for (int k = 1; k < nnb; ++k)
            s += part[k * n + e];
        y[e] = s;
    }
}

}  // namespace ssd
