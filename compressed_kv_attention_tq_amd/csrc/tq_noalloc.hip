// Decode attention for callers that cannot allocate device memory: the chunk
// partials go to a fixed array of the library instead of a caller workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library runs on
// holds its own copy for the life of the process.  In host code its name is only a
// host-side stand-in: the device address of each GPU's copy is looked up once per
// device (hipGetSymbolAddress with that device current) and that address is what
// the kernels receive.  Nothing here calls hipMalloc, hipFree or any allocating
// routine.
#include <atomic>
#include <mutex>

#include "tq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)TQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's copy of the array (looked up on the first
// call on that device), or null on a HIP error.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" tq_status tq_decode_attention_noalloc(const tq_cache *k, const tq_cache *v, const void *q,
                                                 int32_t n_seqs, int32_t n_qtok, int32_t n_q_heads,
                                                 const int32_t *seq_lens, const int32_t *block_table,
                                                 int32_t max_blocks_per_seq, float softmax_scale,
                                                 float sparse_v_tau, float *out, void *stream) {
    // the size this call needs (host-side validation, nothing launched)
    size_t need = 0;
    tq_status st = tq_decode_attention(k, v, q, n_seqs, n_qtok, n_q_heads, seq_lens, block_table,
                                       max_blocks_per_seq, softmax_scale, sparse_v_tau, out, nullptr, &need, stream);
    if (st != TQ_OK) return st;
    if (need > kScratchBytes) return TQ_ERR_WORKSPACE;
    if (n_seqs == 0) return TQ_OK;
    void *ws = device_scratch();
    if (!ws) return TQ_ERR_HIP;
    size_t have = kScratchBytes;
    return tq_decode_attention(k, v, q, n_seqs, n_qtok, n_q_heads, seq_lens, block_table, max_blocks_per_seq,
                               softmax_scale, sparse_v_tau, out, ws, &have, stream);
}
