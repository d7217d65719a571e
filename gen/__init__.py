"""Seeded synthetic inputs shared by the oracle tests and the GPU library's tests and benchmark."""
