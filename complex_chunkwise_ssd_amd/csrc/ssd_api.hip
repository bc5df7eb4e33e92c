// ssd_api.hip -- C ABI of the complex chunkwise SSD scan (declared in
// include/ssd.h): argument checks, work planning and kernel launches on the
// caller's stream. The library allocates nothing.
#include "ssd.h"

#include <ssd_bwd_kernels.h>
#include <ssd_segment_kernels.h>
#include <ssd_mix_kernels.h>

#include <mutex>

// Device scratch of ssd_chunk_forward_noalloc: one copy per GPU, held until the
// process ends. Host code never passes this name to a kernel (on the host it is
// a stand-in, not a device address); it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int launch_status()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

unsigned grid_1d(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

int check_sizes(int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D, int64_t chunk)
{
    if (batch < 0 || T < 0 || H < 0 || N < 1 || D < 1 || chunk < 1)
        return SSD_ERR_SHAPE;
    if (N % 2 != 0)
        return SSD_ERR_ODD_N;
    if (N > SSD_MAX_BLOCK || D > SSD_MAX_BLOCK || chunk > SSD_MAX_BLOCK)
        return SSD_ERR_BLOCK_DIMS;
    // 32-bit token indices, and 32-bit byte offsets inside one chunk of one sequence
    if (T > (1LL << 30) || batch * H > (1LL << 30))
        return SSD_ERR_UNSUPPORTED;
    if (H * (N > D ? N : D) * 8 * 64 > (1LL << 30))
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// The scan over every (sequence, segment, D slice); with several segments, the
// prefix pass (entering states, final state) and the fix-up of the later
// segments' outputs follow on the same stream.
template <int R, int LAYOUT>
int launch_scan(const ssd::ScanParams &base, const ssd::Plan &plan, int64_t seqs, hipStream_t stream)
{
    ssd::ScanParams prm = base;
    prm.groups_per_seq = plan.P;
    const int64_t grid = seqs * plan.P * plan.ndb * plan.nnb;
    hipLaunchKernelGGL((ssd::scan_kernel<R, LAYOUT>), dim3((unsigned)grid),
                       dim3(ssd::kThreads), 0, stream, prm);
    if (int st = launch_status())
        return st;
    if (plan.nnb > 1) {  // add up the N slices' partial outputs
        const int64_t n = (int64_t)prm.B * prm.T * prm.H * prm.D;
        const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
        hipLaunchKernelGGL(ssd::slice_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const float *)prm.y_part, plan.nnb, n, prm.y);
        if (int st = launch_status())
            return st;
    }
    if (plan.P == 1)
        return SSD_OK;
    const int64_t elems = seqs * (int64_t)prm.N * prm.D;
    hipLaunchKernelGGL(ssd::segment_prefix_kernel, dim3(grid_1d(elems, 256)), dim3(256), 0, stream,
                       prm);
    if (int st = launch_status())
        return st;
    const int64_t fix = seqs * (plan.P - 1) * plan.ndb * plan.fix_groups;
    hipLaunchKernelGGL((ssd::segment_fixup_kernel<R, LAYOUT>), dim3((unsigned)fix),
                       dim3(ssd::kFixThreads), 0, stream, prm);
    return launch_status();
}

// Workspace: segment end states, segment log-decays, chunk-start log-decays (with
// several segments) and the N slices' partial outputs (N above 64).
void set_segment_workspace(ssd::ScanParams &prm, const ssd::Plan &plan, void *workspace)
{
    char *w = (char *)workspace;
    if (plan.P > 1) {
        prm.seg_state = (float *)w;
        prm.seg_logdecay = (float *)(w + plan.seg_state_bytes);
        prm.chunk_log = (float *)(w + plan.seg_state_bytes + plan.seg_decay_bytes);
    }
    if (plan.nnb > 1)
        prm.y_part = (float *)(w + plan.seg_state_bytes + plan.seg_decay_bytes +
                               plan.chunk_log_bytes);
    prm.nnb = plan.nnb;
}

template <int LAYOUT>
int launch_forward(const ssd::ScanParams &prm, const ssd::Plan &plan, int64_t seqs,
                   hipStream_t stream)
{
    switch (plan.R) {
    case 16: return launch_scan<16, LAYOUT>(prm, plan, seqs, stream);
    case 32: return launch_scan<32, LAYOUT>(prm, plan, seqs, stream);
    default: return launch_scan<64, LAYOUT>(prm, plan, seqs, stream);
    }
}

template <int R, int LAYOUT, bool SLICED, bool FUSED>
int launch_backward_r(const ssd::BwdParams &prm, int64_t seqs, hipStream_t stream)
{
    const int64_t vseqs = seqs * prm.ns;  // (b, h) x state blocks
    hipLaunchKernelGGL((ssd::bwd_state_kernel<R, false, LAYOUT>), dim3((unsigned)vseqs), dim3(512),
                       0, stream, prm);
    if (int st = launch_status())
        return st;
    if (!FUSED) {  // the fused chunk pass walks the adjoint itself
        hipLaunchKernelGGL((ssd::bwd_state_kernel<R, true, LAYOUT>), dim3((unsigned)vseqs),
                           dim3(512), 0, stream, prm);
        if (int st = launch_status())
            return st;
    }
    const int64_t items = FUSED ? vseqs : vseqs * prm.nc;
    const int64_t groups = items < ssd::kBwdGroups ? items : ssd::kBwdGroups;
    hipLaunchKernelGGL((ssd::bwd_chunk_kernel<R, LAYOUT, SLICED, FUSED>), dim3((unsigned)groups),
                       dim3(512), 0, stream, prm);
    if (int st = launch_status())
        return st;
    if (SLICED) {
        const int64_t n = (int64_t)prm.B * prm.T * prm.H * (prm.D + 2 * prm.N + 1);
        const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
        hipLaunchKernelGGL((ssd::bwd_slice_sum_kernel<LAYOUT>), dim3((unsigned)blocks), dim3(256),
                           0, stream, prm);
        if (int st = launch_status())
            return st;
    }
    // gA shares are laid out (b, h, slice, chunk): ns * nc shares per sequence
    hipLaunchKernelGGL(ssd::bwd_reduce_gA_kernel, dim3((unsigned)prm.H), dim3(256), 0, stream,
                       prm.gA_part, prm.B, prm.H, prm.ns * prm.nc, prm.gA);
    return launch_status();
}

// The fused adjoint walk (any input layout) needs whole sequences per workgroup:
// it is taken when the (virtual) sequences fill the workgroups evenly.
inline bool backward_fused(int64_t vseqs)
{
    return vseqs >= ssd::kBwdGroups && (vseqs % ssd::kBwdGroups == 0 || vseqs >= 4 * ssd::kBwdGroups);
}

template <int R, int LAYOUT>
int launch_backward(const ssd::BwdParams &prm, int64_t seqs, hipStream_t stream)
{
    if (backward_fused(seqs * prm.ns))
        return prm.ns > 1 ? launch_backward_r<R, LAYOUT, true, true>(prm, seqs, stream)
                          : launch_backward_r<R, LAYOUT, false, true>(prm, seqs, stream);
    return prm.ns > 1 ? launch_backward_r<R, LAYOUT, true, false>(prm, seqs, stream)
                      : launch_backward_r<R, LAYOUT, false, false>(prm, seqs, stream);
}

// Workspace carve-up of the backward: stored states and adjoints, gA shares,
// and (state slices) the partial gradients.
void set_backward_workspace(ssd::BwdParams &prm, const ssd::BwdPlan &plan, void *workspace)
{
    char *w = (char *)workspace;
    prm.fwd_states = (float *)w;
    prm.adj_states = (float *)(w + plan.states_bytes);
    prm.gA_part = (float *)(w + 2 * plan.states_bytes);
    char *q = w + 2 * plan.states_bytes + plan.part_bytes;
    prm.gx_part = plan.ns > 1 ? (float *)q : nullptr;
    prm.gB_part = plan.ns > 1 ? (float *)(q + plan.gx_part_bytes) : nullptr;
    prm.gC_part = plan.ns > 1 ? (float *)(q + plan.gx_part_bytes + plan.bc_part_bytes) : nullptr;
    prm.gdt_part = plan.ns > 1 ? (float *)(q + plan.gx_part_bytes + 2 * plan.bc_part_bytes)
                               : nullptr;
    prm.nnb = plan.nnb;
    prm.ndb = plan.ndb;
    prm.ns = plan.ns;
    prm.Q = plan.Q;
    prm.nc = plan.nc;
}

int check_backward_sizes(int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D, int64_t chunk)
{
    if (int st = check_sizes(batch, T, H, N, D, chunk))
        return st;
    // the chunk pass indexes (virtual sequence, chunk) pairs with 32-bit integers
    if (batch > 0 && H > 0 && T > 0) {
        const ssd::BwdPlan plan = ssd::make_bwd_plan(batch, T, H, N, D, chunk);
        if (batch * H * plan.ns * plan.nc >= (1LL << 31))
            return SSD_ERR_UNSUPPORTED;
    }
    return SSD_OK;
}

template <int LAYOUT, class E>
int forward_proj(const E *proj, int64_t token_stride, const ssd_c64 *A, int64_t batch, int64_t T,
                 int64_t H, int64_t N, int64_t D, int64_t chunk_size, const ssd_c64 *initial_state,
                 float *y, ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                 ssd_stream_t stream)
{
    if (int st = check_sizes(batch, T, H, N, D, chunk_size))
        return st;
    if (token_stride < H * (D + 4 * N + 1))
        return SSD_ERR_SHAPE;
    // 32-bit byte offsets inside one chunk of token rows
    if (token_stride > (1LL << 22))
        return SSD_ERR_UNSUPPORTED;
    if (batch == 0 || H == 0)
        return SSD_OK;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!final_state)
            return SSD_OK;
        if (!aligned(final_state, 8) || (initial_state && !aligned(initial_state, 8)))
            return SSD_ERR_ALIGN;
        const int64_t n = batch * H * N * D * 2;
        hipLaunchKernelGGL(ssd::copy_state_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s,
                           (const float *)initial_state, (float *)final_state, n);
        return launch_status();
    }
    if (!proj || !A || !y)
        return SSD_ERR_NULL;
    // B and C are read as pairs of elements: their blocks must start on a pair
    if (!aligned(proj, 2 * sizeof(E)) || token_stride % 2 != 0 || (H * D) % 2 != 0 ||
        !aligned(A, 8) ||
        !aligned(y, 4) || (initial_state && !aligned(initial_state, 8)) ||
        (final_state && !aligned(final_state, 8)))
        return SSD_ERR_ALIGN;
    const ssd::Plan plan = ssd::make_plan(batch, T, H, N, D, chunk_size);
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes)
            return SSD_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return SSD_ERR_ALIGN;
    }
    ssd::ScanParams prm{};
    // element pointers of the row blocks (the kernel reads them as LAYOUT says)
    prm.x = (const float *)proj;
    prm.A = (const float *)A;
    prm.Bt = (const float *)(proj + H * D);
    prm.Ct = (const float *)(proj + H * D + 2 * H * N);
    prm.dt = (const float *)(proj + H * D + 4 * H * N);
    prm.tok_stride = token_stride;
    prm.init_state = (const float *)initial_state;
    prm.y = y;
    prm.final_state = (float *)final_state;
    set_segment_workspace(prm, plan, workspace);
    prm.B = (int)batch;
    prm.T = (int)T;
    prm.H = (int)H;
    prm.N = (int)N;
    prm.D = (int)D;
    prm.Q = (int)ssd::block_rows(chunk_size);
    prm.nc = plan.nc;
    prm.P = plan.P;
    prm.spc = plan.spc;
    prm.ndb = plan.ndb;
    prm.fix_groups = plan.fix_groups;
    return launch_forward<LAYOUT>(prm, plan, batch * H, s);
}

// The backward of the in_proj-row scan; E is the row element (float or the bits
// of a bfloat16), LAYOUT the matching kernel layout.
template <int LAYOUT, class E>
int backward_proj(const E *proj, int64_t token_stride, const ssd_c64 *A, int64_t batch, int64_t T,
                  int64_t H, int64_t N, int64_t D, int64_t chunk_size,
                  const ssd_c64 *initial_state, const float *grad_y,
                  const ssd_c64 *grad_final_state, E *grad_proj, ssd_c64 *grad_A,
                  ssd_c64 *grad_initial_state, void *workspace, size_t workspace_bytes,
                  ssd_stream_t stream)
{
    if (int st = check_backward_sizes(batch, T, H, N, D, chunk_size))
        return st;
    if (token_stride < H * (D + 4 * N + 1))
        return SSD_ERR_SHAPE;
    if (batch == 0 || H == 0)
        return SSD_OK;
    hipStream_t s = (hipStream_t)stream;
    if (!grad_A)
        return SSD_ERR_NULL;
    if (!aligned(grad_A, 8) || (grad_final_state && !aligned(grad_final_state, 8)) ||
        (grad_initial_state && !aligned(grad_initial_state, 8)))
        return SSD_ERR_ALIGN;
    if (T == 0) {
        if (grad_initial_state) {
            const int64_t n = batch * H * N * D * 2;
            hipLaunchKernelGGL(ssd::copy_state_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s,
                               (const float *)grad_final_state, (float *)grad_initial_state, n);
            if (int st = launch_status())
                return st;
        }
        hipLaunchKernelGGL(ssd::bwd_reduce_gA_kernel, dim3((unsigned)H), dim3(256), 0, s,
                           (const float *)nullptr, (int)batch, (int)H, 0, (float *)grad_A);
        return launch_status();
    }
    if (!proj || !A || !grad_y || !grad_proj)
        return SSD_ERR_NULL;
    if (!aligned(proj, sizeof(E)) || !aligned(grad_proj, sizeof(E)) || !aligned(A, 8) ||
        !aligned(grad_y, 4) ||
        (initial_state && !aligned(initial_state, 8)))
        return SSD_ERR_ALIGN;
    const ssd::BwdPlan plan = ssd::make_bwd_plan(batch, T, H, N, D, chunk_size);
    if (!workspace || workspace_bytes < plan.workspace_bytes)
        return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return SSD_ERR_ALIGN;

    const int64_t HD = H * D, HN = H * N;
    // element pointers of the row blocks (the kernels read them as LAYOUT says)
    ssd::BwdParams prm{};
    prm.x = (const float *)proj;
    prm.A = (const float *)A;
    prm.Bt = (const float *)(proj + HD);
    prm.Ct = (const float *)(proj + HD + 2 * HN);
    prm.dt = (const float *)(proj + HD + 4 * HN);
    prm.init = (const float *)initial_state;
    prm.gy = grad_y;
    prm.gfinal = (const float *)grad_final_state;
    prm.gx = (float *)grad_proj;
    prm.gA = (float *)grad_A;
    prm.gB = (float *)(grad_proj + HD);
    prm.gC = (float *)(grad_proj + HD + 2 * HN);
    prm.gdt = (float *)(grad_proj + HD + 4 * HN);
    prm.ginit = (float *)grad_initial_state;
    set_backward_workspace(prm, plan, workspace);
    prm.B = (int)batch;
    prm.T = (int)T;
    prm.H = (int)H;
    prm.N = (int)N;
    prm.D = (int)D;
    prm.Q = plan.Q;
    prm.nc = plan.nc;
    prm.tok_stride = token_stride;
    const int64_t seqs = batch * H;
    return plan.R == 16 ? launch_backward<16, LAYOUT>(prm, seqs, s)
                        : launch_backward<32, LAYOUT>(prm, seqs, s);
}

int check_mix(int64_t tokens, int64_t H, int64_t D)
{
    if (tokens < 0 || H < 1 || D < 1)
        return SSD_ERR_SHAPE;
    if (D > SSD_MAX_BLOCK)
        return SSD_ERR_BLOCK_DIMS;
    if (H * D > ssd::kMixMaxF || tokens > (1LL << 31) - 1)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// True when the np floats at p and the nq floats at q share any byte.
bool overlap(const float *p, int64_t np, const float *q, int64_t nq)
{
    return p && q && np > 0 && nq > 0 && p < q + nq && q < p + np;
}

// Token splits of the gW product: enough workgroups for about one per CU, at
// least kMixMinSplitTokens tokens each; kchunk is the tokens per split.
struct MixSplits {
    int splits, kchunk;
};
MixSplits mix_splits(int64_t tokens, int64_t F)
{
    const int64_t t = (F + ssd::kGemmBM - 1) / ssd::kGemmBM;
    const int64_t tiles = t * t;
    int64_t s = ssd::kMixMaxWorkgroups / tiles;
    const int64_t by_tokens = (tokens + ssd::kMixMinSplitTokens - 1) / ssd::kMixMinSplitTokens;
    s = s < by_tokens ? s : by_tokens;
    s = s < 1 ? 1 : s;
    int64_t kc = (tokens + s - 1) / s;
    kc = (kc + ssd::kGemmBK - 1) / ssd::kGemmBK * ssd::kGemmBK;
    if (kc < ssd::kGemmBK)
        kc = ssd::kGemmBK;
    s = (tokens + kc - 1) / kc;
    return MixSplits{(int)(s < 1 ? 1 : s), (int)kc};
}

template <bool AT, bool BT>
int launch_gemm(const ssd::GemmParams &p, bool vec, hipStream_t stream)
{
    const int64_t groups = (int64_t)p.tiles_m * p.tiles_n * p.splits;
    if (vec)
        hipLaunchKernelGGL((ssd::gemm_kernel<AT, BT, true>), dim3((unsigned)groups),
                           dim3(ssd::kGemmThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((ssd::gemm_kernel<AT, BT, false>), dim3((unsigned)groups),
                           dim3(ssd::kGemmThreads), 0, stream, p);
    return launch_status();
}

// C (M x N) = sum_k A(m, k) B(n, k) over the whole K (one split).
ssd::GemmParams gemm_params(const float *a, int64_t lda, const float *b, int64_t ldb, float *c,
                            int64_t ldc, int64_t M, int64_t N, int64_t K)
{
    ssd::GemmParams p{};
    p.a = a;
    p.b = b;
    p.c = c;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)((M + ssd::kGemmBM - 1) / ssd::kGemmBM);
    p.tiles_n = (int)((N + ssd::kGemmBN - 1) / ssd::kGemmBN);
    p.splits = 1;
    p.kchunk = (int)((K + ssd::kGemmBK - 1) / ssd::kGemmBK * ssd::kGemmBK);
    p.c_split = 0;
    return p;
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return SSD_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_version(void) { return 100; }

const char *ssd_status_string(int status)
{
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid size: negative, or N, D or chunk_size below 1";
    case SSD_ERR_ODD_N: return "N must be even so the complex state packs into real pairs";
    case SSD_ERR_BLOCK_DIMS: return "N, D and chunk_size must not exceed 256";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_ALIGN: return "pointer not aligned as required";
    case SSD_ERR_HIP: return "HIP runtime error";
    case SSD_ERR_UNSUPPORTED:
        return "size not covered by this build (mixer: H * D <= 16384)";
    case SSD_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
    }
}

int ssd_discretise(const float *dt, const ssd_c64 *A, int64_t batch, int64_t T, int64_t H,
                   int64_t chunk_size, ssd_c64 *A_bar, ssd_c64 *log_decay_cumsum,
                   ssd_stream_t stream)
{
    if (batch < 0 || T < 0 || H < 0 || chunk_size < 0)
        return SSD_ERR_SHAPE;
    if (chunk_size > SSD_MAX_BLOCK)
        return SSD_ERR_BLOCK_DIMS;
    if (log_decay_cumsum && chunk_size == 0)
        return SSD_ERR_SHAPE;
    if (batch == 0 || T == 0 || H == 0)
        return SSD_OK;
    if (!dt || !A)
        return SSD_ERR_NULL;
    if (!aligned(dt, 4) || !aligned(A, 8) || (A_bar && !aligned(A_bar, 8)) ||
        (log_decay_cumsum && !aligned(log_decay_cumsum, 8)))
        return SSD_ERR_ALIGN;
    if (batch * T * H > (1LL << 40))
        return SSD_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (A_bar) {
        const int64_t n = batch * T * H;
        hipLaunchKernelGGL(ssd::discretise_abar_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s, dt,
                           (const float *)A, n, (int)H, (float *)A_bar);
        if (int st = launch_status())
            return st;
    }
    if (log_decay_cumsum) {
        const int64_t nc = (T + chunk_size - 1) / chunk_size;
        const int64_t n = batch * nc * H;
        hipLaunchKernelGGL(ssd::discretise_cumsum_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s,
                           dt, (const float *)A, (int)batch, (int)T, (int)H, (int)chunk_size,
                           (int)nc, (float *)log_decay_cumsum);
        if (int st = launch_status())
            return st;
    }
    return SSD_OK;
}

size_t ssd_chunk_forward_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t N,
                                         int64_t D, int64_t chunk_size)
{
    if (check_sizes(batch, T, H, N, D, chunk_size) != SSD_OK || batch == 0 || H == 0 || T == 0)
        return 0;
    return ssd::make_plan(batch, T, H, N, D, chunk_size).workspace_bytes;
}

int ssd_chunk_forward(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t, const ssd_c64 *C_t,
                      const float *dt, int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                      int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                      ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                      ssd_stream_t stream)
{
    if (int st = check_sizes(batch, T, H, N, D, chunk_size))
        return st;
    if (batch == 0 || H == 0)
        return SSD_OK;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!final_state)
            return SSD_OK;
        if (!aligned(final_state, 8) || (initial_state && !aligned(initial_state, 8)))
            return SSD_ERR_ALIGN;
        const int64_t n = batch * H * N * D * 2;
        hipLaunchKernelGGL(ssd::copy_state_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s,
                           (const float *)initial_state, (float *)final_state, n);
        return launch_status();
    }
    if (!x || !A || !B_t || !C_t || !dt || !y)
        return SSD_ERR_NULL;
    if (!aligned(B_t, 8) || !aligned(C_t, 8) || !aligned(x, 8) || !aligned(A, 8) ||
        !aligned(dt, 4) || !aligned(y, 4) || (initial_state && !aligned(initial_state, 8)) ||
        (final_state && !aligned(final_state, 8)))
        return SSD_ERR_ALIGN;

    const ssd::Plan plan = ssd::make_plan(batch, T, H, N, D, chunk_size);
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes)
            return SSD_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return SSD_ERR_ALIGN;
    }

    ssd::ScanParams prm{};
    prm.x = (const float *)x;
    prm.A = (const float *)A;
    prm.Bt = (const float *)B_t;
    prm.Ct = (const float *)C_t;
    prm.dt = dt;
    prm.init_state = (const float *)initial_state;
    prm.y = y;
    prm.final_state = (float *)final_state;
    set_segment_workspace(prm, plan, workspace);
    prm.B = (int)batch;
    prm.T = (int)T;
    prm.H = (int)H;
    prm.N = (int)N;
    prm.D = (int)D;
    prm.Q = (int)ssd::block_rows(chunk_size);
    prm.nc = plan.nc;
    prm.P = plan.P;
    prm.spc = plan.spc;
    prm.ndb = plan.ndb;
    prm.fix_groups = plan.fix_groups;

    return launch_forward<ssd::kLayoutC64>(prm, plan, batch * H, s);
}

int ssd_chunk_forward_noalloc(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t,
                              const ssd_c64 *C_t, const float *dt, int64_t batch, int64_t T,
                              int64_t H, int64_t N, int64_t D, int64_t chunk_size,
                              const ssd_c64 *initial_state, float *y, ssd_c64 *final_state,
                              ssd_stream_t stream)
{
    if (int st = check_sizes(batch, T, H, N, D, chunk_size))
        return st;
    const size_t need = ssd_chunk_forward_workspace_bytes(batch, T, H, N, D, chunk_size);
    if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
        return SSD_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0)
        if (int st = scratch_address(&ws))
            return st;
    return ssd_chunk_forward(x, A, B_t, C_t, dt, batch, T, H, N, D, chunk_size, initial_state, y,
                             final_state, ws, need, stream);
}

int ssd_chunk_forward_proj(const float *proj, int64_t token_stride, const ssd_c64 *A,
                           int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                           int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                           ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                           ssd_stream_t stream)
{
    return forward_proj<ssd::kLayoutProj>(proj, token_stride, A, batch, T, H, N, D, chunk_size,
                                          initial_state, y, final_state, workspace,
                                          workspace_bytes, stream);
}

int ssd_chunk_forward_proj_bf16(const uint16_t *proj, int64_t token_stride, const ssd_c64 *A,
                                int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                                int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                                ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                                ssd_stream_t stream)
{
    return forward_proj<ssd::kLayoutProjBf16>(proj, token_stride, A, batch, T, H, N, D,
                                              chunk_size, initial_state, y, final_state,
                                              workspace, workspace_bytes, stream);
}

size_t ssd_chunk_backward_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t N,
                                          int64_t D, int64_t chunk_size)
{
    if (check_backward_sizes(batch, T, H, N, D, chunk_size) != SSD_OK || batch == 0 || H == 0 ||
        T == 0)
        return 0;
    return ssd::make_bwd_plan(batch, T, H, N, D, chunk_size).workspace_bytes;
}

int ssd_chunk_backward(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t, const ssd_c64 *C_t,
                       const float *dt, int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                       int64_t chunk_size, const ssd_c64 *initial_state, const float *grad_y,
                       const ssd_c64 *grad_final_state, ssd_c64 *grad_x, ssd_c64 *grad_A,
                       ssd_c64 *grad_B_t, ssd_c64 *grad_C_t, float *grad_dt,
                       ssd_c64 *grad_initial_state, void *workspace, size_t workspace_bytes,
                       ssd_stream_t stream)
{
    if (int st = check_backward_sizes(batch, T, H, N, D, chunk_size))
        return st;
    if (batch == 0 || H == 0)
        return SSD_OK;
    hipStream_t s = (hipStream_t)stream;
    if (!grad_A)
        return SSD_ERR_NULL;
    if (!aligned(grad_A, 8) || (grad_final_state && !aligned(grad_final_state, 8)) ||
        (grad_initial_state && !aligned(grad_initial_state, 8)))
        return SSD_ERR_ALIGN;
    if (T == 0) {
        if (grad_initial_state) {
            const int64_t n = batch * H * N * D * 2;
            hipLaunchKernelGGL(ssd::copy_state_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, s,
                               (const float *)grad_final_state, (float *)grad_initial_state, n);
            if (int st = launch_status())
                return st;
        }
        hipLaunchKernelGGL(ssd::bwd_reduce_gA_kernel, dim3((unsigned)H), dim3(256), 0, s,
                           (const float *)nullptr, (int)batch, (int)H, 0, (float *)grad_A);
        return launch_status();
    }
    if (!x || !A || !B_t || !C_t || !dt || !grad_y || !grad_x || !grad_B_t || !grad_C_t ||
        !grad_dt)
        return SSD_ERR_NULL;
    if (!aligned(x, 8) || !aligned(A, 8) || !aligned(B_t, 8) || !aligned(C_t, 8) ||
        !aligned(dt, 4) || !aligned(grad_y, 4) || !aligned(grad_x, 8) || !aligned(grad_B_t, 8) ||
        !aligned(grad_C_t, 8) || !aligned(grad_dt, 4) ||
        (initial_state && !aligned(initial_state, 8)))
        return SSD_ERR_ALIGN;
    const ssd::BwdPlan plan = ssd::make_bwd_plan(batch, T, H, N, D, chunk_size);
    if (!workspace || workspace_bytes < plan.workspace_bytes)
        return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return SSD_ERR_ALIGN;

    ssd::BwdParams prm{};
    prm.x = (const float *)x;
    prm.A = (const float *)A;
    prm.Bt = (const float *)B_t;
    prm.Ct = (const float *)C_t;
    prm.dt = dt;
    prm.init = (const float *)initial_state;
    prm.gy = grad_y;
    prm.gfinal = (const float *)grad_final_state;
    prm.gx = (float *)grad_x;
    prm.gA = (float *)grad_A;
    prm.gB = (float *)grad_B_t;
    prm.gC = (float *)grad_C_t;
    prm.gdt = grad_dt;
    prm.ginit = (float *)grad_initial_state;
    set_backward_workspace(prm, plan, workspace);
    prm.B = (int)batch;
    prm.T = (int)T;
    prm.H = (int)H;
    prm.N = (int)N;
    prm.D = (int)D;
    prm.Q = plan.Q;
    prm.nc = plan.nc;
    const int64_t seqs = batch * H;
    return plan.R == 16 ? launch_backward<16, ssd::kLayoutC64>(prm, seqs, s)
                        : launch_backward<32, ssd::kLayoutC64>(prm, seqs, s);
}

int ssd_chunk_backward_proj(const float *proj, int64_t token_stride, const ssd_c64 *A,
                            int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                            int64_t chunk_size, const ssd_c64 *initial_state, const float *grad_y,
                            const ssd_c64 *grad_final_state, float *grad_proj, ssd_c64 *grad_A,
                            ssd_c64 *grad_initial_state, void *workspace, size_t workspace_bytes,
                            ssd_stream_t stream)
{
    return backward_proj<ssd::kLayoutProj>(proj, token_stride, A, batch, T, H, N, D, chunk_size,
                                           initial_state, grad_y, grad_final_state, grad_proj,
                                           grad_A, grad_initial_state, workspace, workspace_bytes,
                                           stream);
}

int ssd_chunk_backward_proj_bf16(const uint16_t *proj, int64_t token_stride, const ssd_c64 *A,
                                 int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                                 int64_t chunk_size, const ssd_c64 *initial_state,
                                 const float *grad_y, const ssd_c64 *grad_final_state,
                                 uint16_t *grad_proj, ssd_c64 *grad_A,
                                 ssd_c64 *grad_initial_state, void *workspace,
                                 size_t workspace_bytes, ssd_stream_t stream)
{
    return backward_proj<ssd::kLayoutProjBf16>(proj, token_stride, A, batch, T, H, N, D,
                                               chunk_size, initial_state, grad_y,
                                               grad_final_state, grad_proj, grad_A,
                                               grad_initial_state, workspace, workspace_bytes,
                                               stream);
}

int ssd_head_mix(const float *y, const float *W, int64_t tokens, int64_t H, int64_t D, float *z,
                 ssd_stream_t stream)
{
    if (int st = check_mix(tokens, H, D))
        return st;
    if (tokens == 0)
        return SSD_OK;
    if (!y || !W || !z)
        return SSD_ERR_NULL;
    const int64_t F = H * D;
    if (!aligned(y, 4) || !aligned(W, 4) || !aligned(z, 4))
        return SSD_ERR_ALIGN;
    if (overlap(z, tokens * F, y, tokens * F) || overlap(z, tokens * F, W, F * F))
        return SSD_ERR_ALIAS;
    // z = y W^T: A = y (K-contiguous rows), B = W (row o holds output o's weights)
    const ssd::GemmParams p = gemm_params(y, F, W, F, z, F, tokens, F, F);
    const bool vec = F % 4 == 0 && aligned(y, 16) && aligned(W, 16);
    return launch_gemm<false, false>(p, vec, (hipStream_t)stream);
}

size_t ssd_head_mix_backward_workspace_bytes(int64_t tokens, int64_t H, int64_t D)
{
    if (check_mix(tokens, H, D) || tokens == 0)
        return 0;
    const int64_t F = H * D;
    const MixSplits sp = mix_splits(tokens, F);
    if (sp.splits < 2)
        return 0;
    return ssd::align_up((size_t)sp.splits * (size_t)(F * F) * 4, 256);
}

int ssd_head_mix_backward(const float *y, const float *W, const float *grad_z, int64_t tokens,
                          int64_t H, int64_t D, float *grad_y, float *grad_W, void *workspace,
                          size_t workspace_bytes, ssd_stream_t stream)
{
    if (int st = check_mix(tokens, H, D))
        return st;
    if (!grad_W || (tokens > 0 && (!y || !W || !grad_z || !grad_y)))
        return SSD_ERR_NULL;
    if (!aligned(y, 4) || !aligned(W, 4) || !aligned(grad_z, 4) || !aligned(grad_y, 4) ||
        !aligned(grad_W, 4))
        return SSD_ERR_ALIGN;
    const int64_t F = H * D;
    const size_t need = ssd_head_mix_backward_workspace_bytes(tokens, H, D);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return SSD_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 256))
        return SSD_ERR_ALIGN;
    const hipStream_t s = (hipStream_t)stream;
    if (tokens == 0) {  // grad_W = 0
        hipLaunchKernelGGL(ssd::fill_zero_kernel, dim3((unsigned)((F * F + 255) / 256 < 4096 ? (F * F + 255) / 256 : 4096)),
                           dim3(256), 0, s, grad_W, F * F);
        return launch_status();
    }
    const int64_t MF = tokens * F;
    const float *ws = (const float *)workspace;
    const int64_t nws = (int64_t)(need / 4), FF = F * F;
    if (overlap(grad_y, MF, y, MF) || overlap(grad_y, MF, W, FF) || overlap(grad_y, MF, grad_z, MF) ||
        overlap(grad_W, FF, y, MF) || overlap(grad_W, FF, W, FF) || overlap(grad_W, FF, grad_z, MF) ||
        overlap(grad_W, FF, grad_y, MF) || overlap(ws, nws, y, MF) || overlap(ws, nws, grad_z, MF) ||
        overlap(ws, nws, W, FF) || overlap(ws, nws, grad_y, MF) || overlap(ws, nws, grad_W, FF))
        return SSD_ERR_ALIAS;

    // grad_y = gz W: A = gz (K = o contiguous), B(n = k, o) = W[o, k] (transposed)
    const ssd::GemmParams py = gemm_params(grad_z, F, W, F, grad_y, F, tokens, F, F);
    const bool vy = F % 4 == 0 && aligned(grad_z, 16) && aligned(W, 16);
    if (int st = launch_gemm<false, true>(py, vy, s))
        return st;

    // grad_W = gz^T y: A(o, m) = gz[m, o], B(k, m) = y[m, k]; the sum over tokens
    // is cut into splits written to the workspace and added in a fixed order.
    const MixSplits sp = mix_splits(tokens, F);
    ssd::GemmParams pw = gemm_params(grad_z, F, y, F, sp.splits > 1 ? (float *)workspace : grad_W,
                                     F, F, F, tokens);
    pw.splits = sp.splits;
    pw.kchunk = sp.kchunk;
    pw.c_split = F * F;
    const bool vw = F % 4 == 0 && aligned(grad_z, 16) && aligned(y, 16);
    if (int st = launch_gemm<true, true>(pw, vw, s))
        return st;
    if (sp.splits > 1) {
        const int64_t n = F * F;
        const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
        hipLaunchKernelGGL(ssd::split_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           (const float *)workspace, n, sp.splits, n, grad_W);
        return launch_status();
    }
    return SSD_OK;
}

}  // extern "C"
