// Validity count of a top-k selection (the indexer's output that the MHA-prefill code excerpt of
// "DeepSeek-V3.2-Exp · Keys" scatters into the index mask). The attention calls give every entry
// a meaning (outside [0, T): nothing; later than the query: removed by the causal mask; repeated:
// selected once), so nothing in a selection is an error to them; this pass reports how many
// entries fall in each of those cases, and how many queries are left with no allowed key.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

// counts[0]: entries outside [-1, T); counts[1]: entries t with s < t < T; counts[2]: repeats of
// an allowed entry within its row (occurrences after the first); counts[3]: rows whose allowed
// set is empty.
__global__ void check_topk_zero_kernel(unsigned long long* counts) {
    if (threadIdx.x < 4) counts[threadIdx.x] = 0ull;
}

// QR query rows per workgroup: every allowed entry is or-ed into the row's bitmap in LDS, and the
// old word says whether its bit was already set.
template <int QR>
__global__ __launch_bounds__(256) void check_topk_kernel(const int32_t* __restrict__ topk, int T, int K,
                                                         unsigned long long* __restrict__ counts) {
    extern __shared__ uint32_t rows_lds[];    // QR rows of ceil(T/32) words, then QR distinct counts
    const int W = (T + 31) / 32;
    int* distinct = reinterpret_cast<int*>(rows_lds + QR * W);
    const int s0 = blockIdx.x * QR, b = blockIdx.y;
    const int nrows = min(QR, T - s0);
    for (int i = threadIdx.x; i < QR * W + QR; i += 256) rows_lds[i] = 0;
    __syncthreads();
    const int32_t* base = topk + ((size_t)b * T + s0) * K;
    unsigned int bad = 0, late = 0, rep = 0;
    for (int i = threadIdx.x; i < nrows * K; i += 256) {
        const int t = base[i];
        const int qi = i / K;
        const int s = s0 + qi;
        if (t < -1 || t >= T) {
            ++bad;
        } else if (t > s) {
            ++late;
        } else if (t >= 0) {
            const uint32_t bit = 1u << (t & 31);
            const uint32_t old = atomicOr(rows_lds + qi * W + (t >> 5), bit);
            if (old & bit) ++rep; else atomicAdd(distinct + qi, 1);
        }
    }
    __syncthreads();
    unsigned int empty = 0;
    if ((int)threadIdx.x < nrows && distinct[threadIdx.x] == 0) empty = 1;
    // wave sums, one atomic per wave and counter
    auto wsum = [](unsigned int v) {
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        return v;
    };
    bad = wsum(bad);
    late = wsum(late);
    rep = wsum(rep);
    empty = wsum(empty);
    if ((threadIdx.x & 63) == 0) {
        if (bad) atomicAdd(counts + 0, (unsigned long long)bad);
        if (late) atomicAdd(counts + 1, (unsigned long long)late);
        if (rep) atomicAdd(counts + 2, (unsigned long long)rep);
        if (empty) atomicAdd(counts + 3, (unsigned long long)empty);
    }
}

hipError_t launch_check_topk(const int32_t* topk, int B, int T, int K, int64_t* counts, hipStream_t stream) {
    constexpr int QR = 8;
    unsigned long long* c = reinterpret_cast<unsigned long long*>(counts);
    check_topk_zero_kernel<<<1, 64, 0, stream>>>(c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = ((size_t)QR * ((T + 31) / 32) + QR) * sizeof(uint32_t);
    check_topk_kernel<QR><<<dim3((T + QR - 1) / QR, B), 256, lds, stream>>>(topk, T, K, c);
    return hipGetLastError();
}

}  // namespace mla
