// Internal declarations shared by the host and device translation units of
// libs3d8.  Not part of the public ABI.
#ifndef S3D8_INTERNAL_H
#define S3D8_INTERNAL_H

namespace s3d8 {
// Record msg as the calling thread's last error and return code.
int fail(int code, const char *msg);
// Clear the calling thread's last error (called by successful entry points).
void clear_error();
}  // namespace s3d8

#endif
