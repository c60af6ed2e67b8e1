// Row gather / scatter between the caller's per-part buffers and the packed
// layout [P; R_1; ...; R_G] of each group (skillsmp.com "prefix-grouper-grpo",
// "Step 3: Restructure Input Format": the shared prefix once, then the G
// responses back to back; here without padding rows).  A pure HBM copy:
// every byte is read once and written once.

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

constexpr int kRowsThreads = 256;
constexpr int kRowsUnroll = 4;   // chunks per thread, 256 apart
constexpr int kRowsTable = 1024; // groups whose offsets are staged in LDS

// Packed row t of group g (group_start[g] <= t < group_start[g + 1]) is
//   prefix row  t - group_start[g] + prefix_before[g]          if t < prefix_end[g]
//   response row t - prefix_end[g] + group_start[g] - prefix_before[g]  otherwise
// of the caller's prefix / response buffers (prefix_before[g] = prefix rows of
// the groups before g, so group_start[g] - prefix_before[g] is their response
// rows).  Chunks of type C (16 or 4 bytes), `cpr` per row.  kPack: parts ->
// packed, else packed -> parts.
template <typename C, bool kPack>
__global__ __launch_bounds__(kRowsThreads) void rows_kernel(
    const int32_t *__restrict__ gstart, const int32_t *__restrict__ pend,
    const int32_t *__restrict__ pbefore, int ng, C *packed, C *pre, C *resp, long long cpr,
    long long total) {
  __shared__ int32_t s_gs[kRowsTable + 1], s_pe[kRowsTable], s_pb[kRowsTable];
  const bool staged = ng <= kRowsTable;
  if (staged) {
    for (int i = threadIdx.x; i <= ng; i += kRowsThreads) {
      s_gs[i] = gstart[i];
      if (i < ng) {
        s_pe[i] = pend[i];
        s_pb[i] = pbefore[i];
      }
    }
    __syncthreads();
  }
  const int32_t *gs = staged ? s_gs : gstart;
  const int32_t *pe = staged ? s_pe : pend;
  const int32_t *pb = staged ? s_pb : pbefore;
  const long long base = (long long)blockIdx.x * (kRowsThreads * kRowsUnroll) + threadIdx.x;
#pragma unroll
  for (int j = 0; j < kRowsUnroll; ++j) {
    const long long i = base + (long long)j * kRowsThreads;
    if (i >= total) break;
    const long long t = i / cpr, c = i - t * cpr;
    // last group whose start is <= t (empty groups share their start with the next)
    int lo = 0, hi = ng;  // gs[lo] <= t < gs[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (gs[mid] <= t) lo = mid; else hi = mid;
    }
    C *part;
    long long r;
    if (t < pe[lo]) {
      part = pre;
      r = t - gs[lo] + pb[lo];
    } else {
      part = resp;
      r = t - pe[lo] + (gs[lo] - pb[lo]);
    }
    C *a = packed + i;
    C *b = part + r * cpr + c;
    if (kPack) *a = *b; else *b = *a;
  }
}

template <typename C>
hipError_t launch_rows_typed(const Plan &p, bool pack, void *packed, void *pre, void *resp,
                             size_t row_bytes, hipStream_t s) {
  const long long cpr = (long long)(row_bytes / sizeof(C));
  const long long total = (long long)p.T * cpr;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + kRowsThreads * kRowsUnroll - 1) / (kRowsThreads * kRowsUnroll)));
  if (pack)
    hipLaunchKernelGGL((rows_kernel<C, true>), grid, dim3(kRowsThreads), 0, s, p.group_start,
                       p.prefix_end, p.prefix_before, p.n_groups, (C *)packed, (C *)pre,
                       (C *)resp, cpr, total);
  else
    hipLaunchKernelGGL((rows_kernel<C, false>), grid, dim3(kRowsThreads), 0, s, p.group_start,
                       p.prefix_end, p.prefix_before, p.n_groups, (C *)packed, (C *)pre,
                       (C *)resp, cpr, total);
  return hipGetLastError();
}


// Copy of the plan (n16 16-byte chunks) and of the position ids (npos int32)
// from the caller's pinned host staging buffer, read over the bus through its
// device address, into device memory: an ordinary kernel in stream order, so
// the upload needs no hand-off to a copy engine between two kernels.
__global__ __launch_bounds__(256) void upload_kernel(const uint4 *__restrict__ src,
                                                     uint4 *__restrict__ dst, long long n16,
                                                     const uint32_t *__restrict__ psrc,
                                                     uint32_t *__restrict__ pdst,
                                                     long long npos) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < npos; i += stride)
    pdst[i] = psrc[i];
}

}  // namespace

hipError_t launch_rows(const Plan &p, bool pack, void *packed, void *pre, void *resp,
                       size_t row_bytes, hipStream_t s) {
  if (row_bytes % 16 == 0)
    return launch_rows_typed<uint4>(p, pack, packed, pre, resp, row_bytes, s);
  return launch_rows_typed<uint32_t>(p, pack, packed, pre, resp, row_bytes, s);
}

hipError_t launch_upload(const void *src_dev, void *dst, size_t bytes, const void *pos_src_dev,
                         int32_t *pos_dst, size_t npos, hipStream_t s) {
  const long long n16 = (long long)(bytes / 16);
  const long long work = n16 > (long long)npos ? n16 : (long long)npos;
  if (work == 0) return hipSuccess;
  const long long want = (work + 255) / 256;
  const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(upload_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const uint4 *>(src_dev), static_cast<uint4 *>(dst), n16,
                     static_cast<const uint32_t *>(pos_src_dev),
                     reinterpret_cast<uint32_t *>(pos_dst), (long long)npos);
  return hipGetLastError();
}

}  // namespace pg
