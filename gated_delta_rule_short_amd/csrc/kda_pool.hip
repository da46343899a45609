// kda_pool.hip -- copies between rows of a state pool (prefix snapshots, forks).
//
// A pool row holds, per head, the dk x dv state and the head's conv-state
// channels (q, k and v, three taps each).  Source: the state and conv cache of
// "GLM-5.3-Flash im Detail", section "Sequenz-Mixing" (a fixed-size recurrent
// state per head, conv of width four), kept resident for a serving loop that
// reuses cached prefixes ("GLM-5.3-Flash Internals", context-ladder battery).
//
// One workgroup per (copy, head): the state moves as 16-byte pieces with
// non-temporal loads and stores (it is streamed once), the conv rows as
// 16-byte pieces too (a row of 128 channels is 256 or 512 B).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct CopyParams {
    const int32_t *src, *dst;
    const unsigned char *ssrc;
    unsigned char *sdst;
    const unsigned char *csrc;
    unsigned char *cdst;
    int H, num_slots;
    int state_bytes;  // per (slot, head)
    int conv_elem;    // bytes per conv-state element
};

__global__ void __launch_bounds__(256) state_copy_kernel(CopyParams p) {
    constexpr int D = kHeadDim;
    const int H = p.H;
    const int i = blockIdx.x / H, h = blockIdx.x - i * H;
    const int src = pool_slot(p.src, p.num_slots, i), dst = pool_slot(p.dst, p.num_slots, i);
    if (src < 0 || dst < 0 || src == dst) return;
    const int tid = threadIdx.x;
    const u32x4 *s = reinterpret_cast<const u32x4 *>(p.ssrc + ((size_t)src * H + h) * p.state_bytes);
    u32x4 *d = reinterpret_cast<u32x4 *>(p.sdst + ((size_t)dst * H + h) * p.state_bytes);
    // four 16-byte pieces in flight per thread before their stores (the piece count,
    // 4096 for fp32 or 2048 for bf16, is a multiple of 1024)
    const int n = p.state_bytes / 16;
    for (int c = tid; c < n; c += 1024) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(s + c + k * 256);
#pragma unroll
        for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], d + c + k * 256);
    }
    if (!p.csrc) return;
    // conv state [slot][3 taps][CC]: this head's 128 channels of q, k and v per tap
    const int row = D * p.conv_elem, per = row / 16;  // bytes, 16-byte pieces per row
    const size_t CCb = (size_t)3 * H * row;           // bytes of one tap
    for (int c = tid; c < 9 * per; c += 256) {
        const int r = c / per, tap = r / 3, part = r - 3 * tap;
        const size_t off = (size_t)tap * CCb + ((size_t)part * H + h) * row + (size_t)(c - r * per) * 16;
        *reinterpret_cast<u32x4 *>(p.cdst + (size_t)dst * 3 * CCb + off) =
            *reinterpret_cast<const u32x4 *>(p.csrc + (size_t)src * 3 * CCb + off);
    }
}

}  // namespace

hipError_t launch_state_copy(const kda_state_copy_args *a, hipStream_t s) {
    CopyParams p;
    p.src = a->src_slots; p.dst = a->dst_slots;
    p.ssrc = static_cast<const unsigned char *>(a->state_src);
    p.sdst = static_cast<unsigned char *>(a->state_dst);
    p.csrc = static_cast<const unsigned char *>(a->conv_src);
    p.cdst = static_cast<unsigned char *>(a->conv_dst);
    p.H = a->num_heads; p.num_slots = a->num_slots;
    p.state_bytes = kHeadDim * kHeadDim * ((a->flags & KDA_F_STATE_BF16) ? 2 : 4);
    p.conv_elem = a->dtype == KDA_BF16 ? 2 : 4;
    const unsigned blocks = (unsigned)a->count * (unsigned)a->num_heads;
    hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, s, p);
    trace("state_copy_kernel grid=(%u) block=256 lds=0", blocks);
    return hipGetLastError();
}

}  // namespace kda
