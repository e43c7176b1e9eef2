// GPU twin of synth/synth.py: the same seeded synthetic BF16 tensors, bit for
// bit, for workloads too large to draw on the host.  Test and benchmark
// infrastructure; holds none of the quantization arithmetic.  Built with
// -ffp-contract=off so that every float64 operation is rounded exactly as in
// numpy.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;
constexpr uint64_t MUL1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t MUL2 = 0x94D049BB133111EBull;
constexpr uint64_t TAG_ROW = 0x524F57F4C7A1B2C3ull;
constexpr uint64_t TAG_OUT = 0x4F55544C49455221ull;
constexpr double INV_LN2 = 1.4426950408889634;
constexpr double LN2_HI = 0.6931471803691238;
constexpr double LN2_LO = 1.9082149292705877e-10;
constexpr int EXP_TERMS = 14;

__host__ __device__ inline uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * MUL1;
    z = (z ^ (z >> 27)) * MUL2;
    return z ^ (z >> 31);
}

__device__ inline uint64_t draw(uint64_t key, uint64_t counter) { return mix(key + (counter + 1) * GAMMA); }

__device__ inline double irwin_hall12(uint64_t key, uint64_t idx) {
    uint64_t total = 0;
    for (int j = 0; j < 6; j++) {
        uint64_t d = draw(key, idx * 6 + j);
        total += (d >> 32) + (d & 0xFFFFFFFFull);
    }
    int64_t centred = (int64_t)total - (int64_t)(6ull << 32);
    return (double)centred * 0x1p-32;
}

__device__ inline double exp_det(double y) {
    double k = rint(y * INV_LN2);
    double f = (y - k * LN2_HI) - k * LN2_LO;
    double p = 1.0;
    for (int n = EXP_TERMS; n > 0; n--) p = 1.0 + (f / (double)n) * p;
    return ldexp(p, (int)k);
}

__global__ void k_fill(uint16_t* out, int64_t M, int64_t N, uint64_t key, uint64_t rkey, uint64_t okey,
                       double sigma, double row_sigma, double outlier_p, double outlier_factor) {
    const int64_t total = M * N;
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= total) return;
    int64_t row = -1;
    double rowf = 1.0;
    for (int k = 0; k < 8 && i0 + k < total; k++) {
        const int64_t i = i0 + k;
        const int64_t r = i / N;
        if (r != row) {
            row = r;
            rowf = row_sigma == 0.0 ? 1.0 : exp_det(row_sigma * irwin_hall12(rkey, (uint64_t)r));
        }
        double w = (sigma * irwin_hall12(key, (uint64_t)i)) * rowf;
        if (outlier_p > 0.0) {
            double u = (double)(draw(okey, (uint64_t)i) >> 11) * 0x1p-53;
            w = w * (u < outlier_p ? outlier_factor : 1.0);
        }
        float f = (float)w;
        uint32_t b = __float_as_uint(f);
        out[i] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    }
}

}  // namespace

extern "C" int synth_fill_bf16(uint16_t* out, int64_t M, int64_t N, uint64_t seed, uint64_t stream_id, double sigma,
                               double row_sigma, double outlier_p, double outlier_factor, void* hip_stream) {
    if (!out || M <= 0 || N <= 0) return 1;
    const uint64_t key = mix(seed * GAMMA + stream_id);
    const int64_t threads = (M * N + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, out, M, N, key,
                       mix(key ^ TAG_ROW), mix(key ^ TAG_OUT), sigma, row_sigma, outlier_p, outlier_factor);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
